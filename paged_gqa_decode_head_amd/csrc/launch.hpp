// Internal launch interface between the C ABI layer (api.cpp) and the kernels.
// Arguments are validated by the caller; these functions only enqueue.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pgqa {

// Physical layout of one pool: for block b and kv head g the (b, g) tile holds
// K row-major [block_size][128] and then V transposed [128][block_size], bf16.
struct PoolGeom {
  uint16_t* kv;          // device base
  int32_t num_blocks;
  int32_t block_size;
  int32_t num_kv_heads;
  uint32_t* err;         // device sticky error word
};

__host__ __device__ inline int64_t tile_elems(const PoolGeom& p) { return 2ll * p.block_size * 128; }

// Inside one (block, kv head) tile: K row-major [slot][128], then V transposed
// in 16-slot pieces [slot / 16][128][16], so that 16 consecutive keys of V^T are
// one contiguous 4 KiB run (whole 128-byte lines) at every block size.
constexpr int kVSub = 16;  // slots per V^T piece
__host__ __device__ inline int64_t v_elem(int bs, int slot, int dim) {
  return (int64_t(bs) << 7) + (int64_t(slot >> 4) << 11) + dim * kVSub + (slot & (kVSub - 1));
}

struct WriteArgs {
  const uint16_t* q; int64_t q_stride;
  const uint16_t* k; int64_t k_stride;
  const uint16_t* v; int64_t v_stride;
  const uint16_t* wq; const uint16_t* wk;
  const int32_t* pos; const int32_t* seq;
  const int32_t* bt; int32_t bt_stride; int32_t num_seqs;
  int32_t num_tokens; int32_t num_q_heads;
  float eps;
  double rev_freq[64];   // theta^(-2i/128) / (2 pi): turns per position of rotary pair i
  uint16_t* q_out;
};

hipError_t launch_cache_write(const PoolGeom& pool, const WriteArgs& a, hipStream_t stream);

struct DecodeArgs {
  const uint16_t* q; int64_t q_stride;  // q row stride per sequence (query token for chunk segments), elements
  const int32_t* ctx;
  const int32_t* bt; int32_t bt_stride;
  int32_t batch; int32_t num_q_heads; int32_t max_ctx;
  float qk_scale_log2;   // softmax scale * log2(e)
  int32_t split_tokens; int32_t max_splits; int32_t waves;
  int32_t mfma;          // 1: matrix-core split kernel, 0: dot-product split kernel
  int32_t stream_loads;  // 1: K/V loads carry the non-temporal (streaming) hint
  float* part_o;         // [batch][Hkv][max_splits][r][128] (chunk segments: 16 columns instead of r)
  float* part_lse;       // [batch][Hkv][max_splits][r]
  uint16_t* out;         // [batch][Hq][128] (chunk segments: [total_q][Hq][128], row stride q_stride)
  // Chunk segments on the matrix-core kernel (launch_decode_columns): batch
  // counts segments, whose query rows start at qsl[b]; nullptr otherwise.
  const int32_t* qsl; int32_t total_q; int32_t max_q_len;
};

// The fused decode step (norm + rotary of the new token's q and k, its cache
// write, and decode attention in one launch): raw rows of the one new token of
// each sequence, at position context_len - 1.
struct StepArgs {
  const uint16_t* k; int64_t k_stride;
  const uint16_t* v; int64_t v_stride;
  const uint16_t* wq; const uint16_t* wk;
  float eps;
  uint16_t* q_out;       // optional: the normed, rotated q (bf16 [batch][Hq][128])
  double rev_freq[64];   // theta^(-2i/128) / (2 pi): turns per position of rotary pair i
};

// Optional order of the decode grid's (sequence, kv head) units, passed by
// value as a kernel argument: position p = sequence * Hkv + kv head of the grid
// computes unit unit[p] instead (count == 0: natural order).  Built on the host
// from host-side context lengths so that long and short units share a CU.
constexpr int kMaxOrderedUnits = 1024;
struct UnitOrder {
  int32_t count;
  uint16_t unit[kMaxOrderedUnits];
};

// st == nullptr: plain decode attention over q as given; ord == nullptr: natural unit order.
hipError_t launch_decode(const PoolGeom& pool, const DecodeArgs& a, const StepArgs* st, const UnitOrder* ord,
                         hipStream_t stream);

// Chunk segments of at most 16 query rows (q_len x group) per kv head on the
// matrix-core decode kernel, one workgroup per (kv head, segment, split).
hipError_t launch_decode_columns(const PoolGeom& pool, const DecodeArgs& a, hipStream_t stream);

// The allocation-free decode step keeps its split partials in a fixed device
// array of kNoAllocScratchBytes per GPU.  noalloc_scratch returns that array's
// address on the current device (looked up once per device, thread-safe).
constexpr size_t kNoAllocScratchBytes = size_t(8) << 20;
hipError_t noalloc_scratch(void** ptr);

// Workspace carve-up shared by the host API and the launchers.
struct DecodeWorkspace {
  size_t part_o_off, part_lse_off, total;  // total = 0 when max_splits == 1
};
DecodeWorkspace decode_workspace_layout(int32_t batch, int32_t num_kv_heads, int32_t group, int32_t max_splits);

struct ChunkArgs {
  const uint16_t* q;
  const int32_t* qsl; const int32_t* ctx;
  const int32_t* bt; int32_t bt_stride;
  int32_t num_segments; int32_t total_q; int32_t num_q_heads;
  int32_t max_q_len; int32_t max_ctx;
  float qk_scale_log2;
  int32_t split_wide;    // keys per split, segments of more than 32 rows per kv head
  int32_t split_short;   // keys per split, segments of at most 32 rows per kv head
  int32_t max_splits;    // partial slots per row: covers both split sizes
  float* part_o;         // [max_splits][total_q][Hq][128]
  float* part_lse;       // [max_splits][total_q][Hq]
  uint16_t* out;
  // Mixed-step calls (launch_mixed): the host-built work list, kMixedItemInts
  // int32 per item, num_items attention items followed by the combine items;
  // split_short is then the key split of the query-column items.
  const int32_t* items;
  int32_t num_items;
};

// Which chunk work lists a call can have: wide (segments of more than 32 rows
// per kv head) if some segment may be that long (a lone segment holds all
// total_q tokens), short unless a lone segment is longer.
struct ChunkLists {
  bool wide, narrow;
};
inline ChunkLists chunk_lists(int32_t num_segments, int32_t total_q, int32_t group, int32_t max_q_len) {
  const bool lone_wide = num_segments == 1 && int64_t(total_q) * group > 32;
  return ChunkLists{int64_t(max_q_len) * group > 32 || lone_wide, !lone_wide};
}

// Grid sizes (upper bounds of the device-side work lists) of the chunk kernels.
struct ChunkGrids {
  int64_t wide, narrow, combine;
};
ChunkGrids chunk_grids(int32_t num_segments, int32_t total_q, int32_t num_kv_heads, int32_t group, int32_t max_q_len,
                       int32_t max_ctx, int32_t split_wide, int32_t split_short, int32_t max_splits);

hipError_t launch_chunk(const PoolGeom& pool, const ChunkArgs& a, const ChunkGrids& grids, hipStream_t stream);

// One attention launch (and one combine launch when num_combine > 0) for a
// mixed step from a host-built work list (items of kMixedItemInts int32:
// segment, kind, kv head, row group or first combine row, split or split count,
// and the host's query offset, query length and key count of the segment).
constexpr int kMixedItemInts = 8;
hipError_t launch_mixed(const PoolGeom& pool, const ChunkArgs& a, int32_t num_combine, hipStream_t stream);

// Plain streaming read of words16 16-byte words (the achievable-bandwidth reference).
hipError_t launch_stream_read(const void* src, int64_t words16, void* sink, int grid, hipStream_t stream);

struct ChunkWorkspace {
  size_t part_o_off, part_lse_off, total;  // total = 0 when max_splits == 1
};
ChunkWorkspace chunk_workspace_layout(int32_t total_q, int32_t num_q_heads, int32_t max_splits);

}  // namespace pgqa
