/* actsparse_timeline.h -- phase timelines of the sparse SwiGLU MLP and of the
 * decode attention.
 *
 * Declared only for libactsparse_timeline.so, the opt-in build of libactsparse
 * made by `python -m activation_sparse_gemv_amd.build --timeline` (the kernels
 * compiled with AS_PHASE_TIMELINE).  libactsparse.so does not export it: its
 * kernels carry no timeline code.
 *
 * The timeline shows where a one-token MLP layer spends its time inside the two
 * row-gather launches (gate/up, then down): each workgroup's thread 0 writes the
 * device's 100 MHz constant clock at its phase boundaries.  It measures the fused
 * mask-plus-gather design of the TEAL slides (slide 11, the kernel that tests
 * |x_i| > t and streams only the kept weight rows) on this chip.
 */
#ifndef ACTSPARSE_TIMELINE_H
#define ACTSPARSE_TIMELINE_H

#include <stddef.h>
#include <stdint.h>

#include "actsparse.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Arms a timeline buffer for the next as_sparse_swiglu_mlp call made on any
 * thread of the process (that call disarms it).
 *   buf    device memory of `words` 64-bit words, zeroed by the caller; the call
 *          writes workgroup g of the gate/up launch at buf[16*g ...] and workgroup
 *          g of the down launch at buf[words/2 + 16*g ...]; a launch whose grid
 *          needs more than words/2 words is not recorded.
 *   Slots of a workgroup's 16 words (times in 10 ns ticks; 0: not reached):
 *     0 entry; 1 prologue done (rows listed in LDS); 2 main loop done;
 *     3 slot reduction done; 4 partial tile stored and complete; 5 tile counter
 *     returned; 6 output written (last workgroup of a column tile);
 *     7 rows gathered (a count); 8 prologue input arrived; 9 prologue scan done
 *     (gate/up) or SwiGLU staged (down); 10 h exports done (down); 11 split
 *     points of the row list (gate/up); 12 row list written by thread 0's wave;
 *     13 barrier after the row list passed (gate/up).
 * Returns AS_ERR_INVALID_ARG for a NULL buffer or words < 32.  The buffer is owned
 * by the caller and must stay valid until the armed call's launches complete. */
as_status as_phase_timeline_arm(uint64_t* buf, size_t words);

/* Arms a timeline buffer for the next as_gqa_decode_attention call (the decoder
 * block's attention launch included) made on any thread of the process; that call
 * disarms it.  Workgroup (kv head g, chunk c) of a grid of n_kv x C writes its 16
 * words at buf[16 * (g + n_kv * c) ...]; a grid needing more than `words` words is
 * not recorded.  Slots (10 ns ticks; 0: not reached): 0 entry; 1 scores computed
 * (query and K rows arrived); 2 chunk maximum known (first barrier passed); 3 wave
 * partial outputs in LDS (second barrier passed); 4 chunk record stored and
 * complete; 5 arrival counter returned; for the last chunk of a kv head only:
 * 6 merge weights ready (statistics loaded, third barrier passed); 7 output
 * stored.  Errors and ownership as for as_phase_timeline_arm. */
as_status as_attention_timeline_arm(uint64_t* buf, size_t words);

#ifdef __cplusplus
}
#endif

#endif /* ACTSPARSE_TIMELINE_H */
