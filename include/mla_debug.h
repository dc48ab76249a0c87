/*
 * mla_debug.h -- extra C ABI of libmla_phases.so, the instrumented build of
 * libmla (the same sources compiled with -DMLA_PHASE_STAMPS).  Every entry
 * point of include/mla.h behaves as in libmla.so; in addition, each wave of
 * the bf16 split-KV kernel (split_kv_ring_kernel) keeps lap timers in shader
 * cycles that this call reads back.  libmla.so does not export it.  The
 * timers cost a few scalar instructions and a wait per lap, so the
 * instrumented build runs slightly slower than libmla.so.
 */
#ifndef MLA_DEBUG_H
#define MLA_DEBUG_H

#include <stddef.h>

#include "mla.h"

#ifdef __cplusplus
extern "C" {
#endif

/* 256 workgroups x 4 waves x 16 words. */
#define MLA_PHASE_WORDS 16384

/*
 * Waits for the device, copies the timers (MLA_PHASE_WORDS unsigned 32-bit
 * words) to host_dst and clears them.  Word 16 (4 b + w) + k belongs to wave
 * w of workgroup b of the last bf16 split-KV launch (each launch overwrites
 * the words of its working waves); a workgroup with no piece leaves zeros.
 *   k = 0, 1, 2   steady-state half-tiles: barrier wait, score chain, value
 *                 chain (softmax threaded in), cycles summed over them
 *   k = 3         number of steady-state half-tiles
 *   k = 4         the wave's cycles, start to end
 *   k = 5         pieces processed
 *   k = 6, 7      low 32 bits of the 100 MHz real-time counter at the
 *                 wave's start and end
 *   k = 8         kernel start (or previous piece's end) to the piece's
 *                 start: the schedule walk
 *   k = 9         to the piece's first half-tile landed (block table,
 *                 query fragments, first copies)
 *   k = 10        the first half-tile's scores and softmax
 *   k = 12        the piece's last two half-tiles and its final value chain
 *   k = 13        the vote on the softmax reference (and any repeated pass)
 *   k = 14        the epilogue: partial o_lat and log-sum-exp written
 *   k = 11, 15    zero
 * Words 0-2 and 8-14 of a wave sum to word 4.
 * Returns MLA_ERR_NULL_POINTER, MLA_ERR_BAD_SHAPE (bytes is not
 * 4 * MLA_PHASE_WORDS) or MLA_ERR_HIP; MLA_OK otherwise.
 */
mla_status mla_debug_phase_stamps(void* host_dst, size_t bytes);

#ifdef __cplusplus
}
#endif

#endif /* MLA_DEBUG_H */
