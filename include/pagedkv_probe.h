/*
 * pagedkv_probe — a measurement aid exported by libpagedkv.so, outside the
 * attention path.
 *
 * Decode attention over a paged cache is a stream of reads of whole
 * (block, kv-head) tiles at the physical block positions a block table
 * names ("LLM Engineering (5)": "Two phases with very different
 * characteristics" for the whole-cache read of every step, "Paged
 * attention" for the fixed-size blocks).  This probe performs only that
 * read pattern, with no arithmetic beyond folding the bytes into a sink, so
 * the rate the device sustains for it can be measured on the same GPU and
 * the decode kernel's rate stated as a fraction of it.
 */
#ifndef PAGEDKV_PROBE_H
#define PAGEDKV_PROBE_H

#include "pagedkv.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Tile-gather read.  Reads the num_tiles 4096-byte tiles
 *   pool + 4096 * tile_ids[i],   i in [0, num_tiles)
 * once each (16-byte loads, whole tiles per wave, four tiles in flight per
 * wave) and writes one 32-bit xor fold per thread to sink.
 *   pool      device, caller-owned; 4096-byte aligned
 *   tile_ids  device int32 [num_tiles]; every id must name a tile inside
 *             pool (not checked: an id out of range is a memory fault)
 *   num_tiles >= 0 (0: no launch)
 *   grid      workgroups of 256 threads, in [1, 65536]
 *   streaming 0: the default load policy; 1: loads with the non-temporal
 *             hint, as decode issues them over a cache pool for which
 *             pkv_paged_attention_streams_cache returns 1
 *   sink      device uint32 [grid * 256], caller-owned, overwritten
 *   stream    hipStream_t as void*, NULL = default stream
 * Returns PKV_ERR_INVALID (nothing launched) for a null pointer, a
 * misaligned pool, num_tiles < 0, grid out of range or streaming not 0 or
 * 1; PKV_ERR_HIP if the launch fails.
 */
pkv_status pkv_probe_tile_read(const void* pool, const int32_t* tile_ids, int64_t num_tiles,
                               int32_t grid, int32_t streaming, uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDKV_PROBE_H */
