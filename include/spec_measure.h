/*
 * spec_measure.h -- measurement hooks of libspecverify.so.
 *
 * Not part of the verification method: these calls exist so that a benchmark
 * can time each library kernel with HIP events on the stream it runs on, and
 * can calibrate bandwidth figures against plain streaming kernels.
 */
#ifndef SPEC_MEASURE_H
#define SPEC_MEASURE_H

#include <stddef.h>
#include <stdint.h>

#include "spec_verify.h"

#ifdef __cplusplus
extern "C" {
#endif

/* While enabled, every kernel the library launches is bracketed by a pair of
 * HIP events recorded on its launch stream.  Process-wide; not for use while
 * other threads call the library.  Enabling creates events (host allocation). */
spec_status_t spec_timing_enable(int enable);

/* Drop every recorded launch. */
spec_status_t spec_timing_reset(void);

/* Waits for the recorded events, then aggregates them per kernel name.
 * Returns the number of distinct kernel names recorded since the last reset. */
int spec_timing_collect(void);

/* Entry `index` (0 <= index < spec_timing_collect()) of the aggregate:
 * kernel name (static storage), number of launches, summed milliseconds. */
spec_status_t spec_timing_entry(int index, const char** name, long long* launches, double* total_ms);

/* Process-wide overrides of choices the library otherwise makes itself, for tests
 * and measurements.  Each knob starts at its default; spec_set_knob with a negative
 * value restores it.  Set knobs only while no call of the library is being issued on
 * another thread; a call reads every knob once, when it is issued.
 *
 *   SPEC_KNOB_CHUNK_VECTORS  16-byte vectors per lane in one chunk of the streaming
 *                            passes (chain row statistics, tree row argmax): 1, 2, 4,
 *                            8 or 16 (16 only for bf16 chain rows with 16-byte loads);
 *                            0 (default) = the library's choice.
 *   SPEC_KNOB_POLL_LIMIT     polls of a hand-over word that has not arrived before a
 *                            cross-workgroup wait gives up and flags its sequence -2
 *                            (default 262144, at least a quarter of a second); 0 = give
 *                            up before the first poll, so that every sequence that needs
 *                            a wait is flagged (a test of the flag path).
 *   SPEC_KNOB_SINGLE_LAUNCH  0 (default): spec_verify_chain and spec_ngram_verify run as one
 *                            launch (plus the packed output's) when the whole grid fits on
 *                            the device at once; 1: always as separate statistics and
 *                            draw launches.
 *   SPEC_KNOB_XCD_LOCAL      1 (default): where all workgroups of a sequence run on one XCD
 *                            (the fused chain launch, the pool kernel and the tree walks of a
 *                            batch, or of a launch's share of it, whose size is a multiple of
 *                            8; the single chain launch of 8 sequences or more), the values
 *                            they hand each other go through that XCD's L2; 0: every
 *                            hand-over through agent-scope stores, in the spread placement.
 *                            The results are the same either way.
 */
typedef enum spec_knob {
  SPEC_KNOB_CHUNK_VECTORS = 0,
  SPEC_KNOB_POLL_LIMIT = 1,
  SPEC_KNOB_SINGLE_LAUNCH = 2,
  SPEC_KNOB_XCD_LOCAL = 3
} spec_knob_t;

spec_status_t spec_set_knob(spec_knob_t knob, int value);

/* Current value of a knob (its default unless set), or -1 for an unknown knob. */
int spec_get_knob(spec_knob_t knob);

/* Phase timestamps of spec_verify_chain's kernels.  While `buffer` (device memory of
 * `words` unsigned 64-bit words) is set, every following call whose stamps fit writes
 * the device's constant 100 MHz clock at its phase boundaries into it (a call that needs
 * more words writes none): with G = B * R * C stats workgroups (R rows and C chunks per
 * row as the call chose them) and P pool tasks (task t = b * CP + c is task c of the CP
 * of sequence b), words [2g, 2g+1] are the start and end of
 * stats workgroup g and words [2G + 6t, 2G + 6t + 5] those of pool task t: start,
 * decision made, own segment masses published (or the piece chosen, for a draw from a
 * target row), siblings' masses gathered (the waiting task), end, and
 * (b << 32) | (c << 8) | mode.  A call that runs as one launch (SPEC_KNOB_SINGLE_LAUNCH)
 * stamps its B * (K+1) * C workgroups of sequences instead (w = (b * (K+1) + k) * C + c,
 * the lookup's workgroups unstamped): words [6w, 6w + 5] are its start, its partials
 * published, every partial gathered, decision made, draw located (or own segment masses
 * published) and end.  A call that runs as the fused launch (statistics and draws in one
 * launch, with CP helper workgroups a sequence) stamps words [2g, 2g+1] for stats chunk g in
 * (sequence, row, chunk) order (start, partials published), then four words per sequence b
 * from 2G + 4b (its finisher's partials gathered, decision published, end, and the decision's
 * mode), then seven words per helper h = b * CP + c from 2G + 4B + 7h (start, decision seen,
 * own segment masses published, draw located, drawn segment narrowed and the row written,
 * exit, and, in a residual draw, (b << 32) | (c << 8) | n with n = 1 for the helper that
 * narrowed, 0 for the others).  Words of phases a task
 * does not reach are left as they were.  NULL stops the stamping.  Measurement only; the same
 * thread rule as the knobs. */
spec_status_t spec_chain_phase_stamps(unsigned long long* buffer, size_t words);

/* Read-only streaming probe in the access shape of the library's streaming passes: one
 * workgroup per `chunk_bytes` chunk (16384, 32768 or 65536), chunks dealt to the XCDs in
 * contiguous blocks, each wave reading one contiguous quarter of its chunk with
 * non-temporal 16-byte loads.  `bytes` is a whole number of chunks at a 16-byte aligned
 * `src`; *out (device uint32) is written only in a case that never occurs (it keeps the
 * loads alive).  The figure it gives is the achievable read rate the streaming passes are
 * compared with. */
spec_status_t spec_probe_read(const void* src, size_t bytes, size_t chunk_bytes, uint32_t* out,
                              spec_stream_t stream);

/* Plain copy of `bytes` (a multiple of 16, 16-byte aligned) from src to dst. */
spec_status_t spec_probe_copy(const void* src, void* dst, size_t bytes, spec_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* SPEC_MEASURE_H */
