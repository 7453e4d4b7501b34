/*
 * mfl_probe.h — test-only entry points of the MI355X fp16 GEMM library.
 *
 * They exist so tests can pin hardware facts the pages cannot: which lane and
 * register slot of a gfx950 matrix instruction holds which matrix element
 * (the role the SM80 thread/value tables play on the TiledMMA page
 * "读懂 CuTe 的 make_tiled_mma", section "从 C 的四个值开始读").
 */
#ifndef MFL_PROBE_H
#define MFL_PROBE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* One wave (64 lanes) issues one matrix instruction `op` (numbering as
 * mfl_layout_mfma_tv).  Lane l takes A slots a_slots[l*VA .. l*VA+VA) and B
 * slots b_slots[l*VA ..] (fp16 bit patterns, VA = 8 for ops 0,1 and 4 for
 * ops 2,3) and accumulator inputs c_slots[l*VC .. +VC) (fp32, VC = 16 for the
 * 32x32 ops, 4 for the 16x16 ops); it writes its accumulator outputs to
 * d_out[l*VC .. +VC).  All four pointers are device memory sized 64*VA or
 * 64*VC elements.  Enqueued on `stream` (a hipStream_t).  Returns 0, -4 for
 * a bad op or NULL pointer, -5 on a launch error. */
int mfl_probe_mfma(int32_t op, const uint16_t* a_slots, const uint16_t* b_slots,
                   const float* c_slots, float* d_out, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* MFL_PROBE_H */
