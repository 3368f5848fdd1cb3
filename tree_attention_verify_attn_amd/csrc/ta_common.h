// Definitions shared by the host entry points and the gfx950 kernels of the
// split tree-verify attention library.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace ta {

constexpr int kBlock = 64;        // tokens per KV-cache block
constexpr int kThreads = 256;     // threads per workgroup of the small kernels (4 wave64)
constexpr int kAttnThreads = 512; // threads per workgroup of the attention kernel (8 wave64)
constexpr int kAttnWaves = kAttnThreads / 64;
constexpr int kMaxTree = 64;      // fused kernel and commit: one 64-bit mask word per tree node
constexpr int kMaxTreeSplit = 256; // split path: up to four mask words per tree node
constexpr int kMaxBatch = 2048;   // per-workgroup item table lives in LDS
constexpr int kRowsPerPass = 64;  // grouped query rows one work item covers
constexpr int kMaxSplits = 64;    // cap on work items per (sequence, head, row pass)
// One-sequence launches whose groups have at least this many chunks end the
// attention kernel at the partial stores and combine in a second launch.
constexpr int kTwoLaunchMinChunks = 2;
// Short prefixes stream in one chunk per sequence, with no exchange at all:
// one sequence up to this many blocks (against two launches of 64-token
// chunks), a batch whose longest prefix has up to kOneChunkBlocksBatch
// (against chunks that meet in the launch), or up to kOneChunkBlocksWide
// when at least kOneChunkWideGroups groups (sequence, KV head, row pass)
// share the launch and splitting would add many meetings.
constexpr int kOneChunkBlocks = 3;
constexpr int kOneChunkBlocksBatch = 6;
constexpr int kOneChunkBlocksWide = 8;
constexpr int kOneChunkWideGroups = 32;
constexpr unsigned kSpinLimit = 1u << 22;
constexpr int kLdsBytes = 160 * 1024;  // LDS per CU (gfx950)
constexpr int kMaxRingSlots = 2;       // KV blocks the attention kernel keeps in LDS
constexpr int kMaxChunk = 4096;        // prefix tokens per work item, at most

// Status codes, identical to ta_status in include/tree_attn.h.
enum : int {
  kOk = 0,
  kErrInvalidArg = 1,
  kErrUnsupported = 2,
  kErrBadTree = 3,
  kErrWorkspace = 4,
  kErrHip = 5,
  kErrBadPrefix = 6,
  kErrTimeout = 7,
  kErrNoBlocks = 8,
  kErrScratch = 9,
};

constexpr int kCounterStride = 64;  // unsigned words between two counters: one 256-byte line each
// words of a group's line in the barrier region: arrival counter at 0, then
constexpr int kStartedWord = 8;     // chunks of the group that have started
constexpr int kLeaveWord = 16;      // 64-bit mask of chunks that left without waiting
constexpr int kSenseWord = 32;      // sense word the waiting chunks poll
constexpr int kBarrierSlots = 1024; // group barriers in the workspace's fixed region (grid size bound)
constexpr int kMaxGroups = 1 << 18; // ticket arrival counters: batch * kv heads * row passes, at most

// First 768 bytes of every workspace: each field on a cache line of its own,
// so that the device-scope atomics on one do not queue behind those on another.
struct WsHeader {
  int error;          // first device-detected error code (0 = none)
  unsigned pad0[kCounterStride - 1];
  unsigned done;      // workgroups that have left the persistent loop
  unsigned pad1[kCounterStride - 1];
  unsigned ticket;    // next dynamically assigned work item (minus the first round)
  unsigned pad2[kCounterStride - 1];
};
static_assert(sizeof(WsHeader) == 3 * 4 * kCounterStride, "workspace header layout");

// Everything a kernel needs for one call.  Built on the host, passed by value.
//
// Work decomposition of the prefix pass.  A group is (sequence b, KV head g,
// row pass rp); its prefix is cut into chunks of `chunk` tokens, one work item
// each.  Items are numbered densely, sequence by sequence, then KV head, row
// pass and chunk (chunk fastest), from a table of the sequences every
// workgroup builds in LDS; the chunks of a group have consecutive numbers.
// Workgroup i first takes item i, then items from one device-wide ticket
// counter, in increasing order.  The chunk partials of a group are exchanged
// through device-coherent (L2-bypassing) accesses, so a group may span XCDs.
struct Params {
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_table;
  const int32_t* prefix_lens;
  const void* k_tree;
  const void* v_tree;
  const int32_t* parents;
  const int32_t* tree_offsets;
  const uint64_t* mask_in;   // suffix kernel input (split path)
  void* out;                 // fused: shape dtype;  prefix/suffix: fp32
  float* lse_out;            // may be null in fused mode
  WsHeader* hdr;
  unsigned* arrive;          // [kBarrierSlots] (arrival counter, sense) pairs, kCounterStride
                             // apart, then [kMaxGroups] ticket arrival counters
  float* partials;           // [item slots][slot_floats]
  int batch, hq, hkv, group, head_dim;
  int max_blocks, max_tree, max_prefix, total_nodes, num_blocks;
  int mask_words;            // 64-bit mask words per tree node: cdiv(max_tree, 64)
  int chunk;                 // prefix tokens per work item (multiple of 64)
  int rp_max;                // row passes per (sequence, head)
  int rows_slot;             // rows reserved per partial slot
  int slot_floats;           // floats per partial slot
  int num_groups;            // batch * hkv * rp_max
  int s_max;                 // chunks per group, upper bound
  int item_slots;            // num_groups * s_max: bound on item numbers
  int chunk_auto;            // 1: the kernel may pick the chunk from the actual prefix lengths
  int tree_in_cache;         // 1: tree K/V rows are cache positions P .. P+T-1 (k_tree unused)
  int single;                // 1: one sequence, items numbered without a table
  int single_items;          // item count of a one-sequence launch
  int xcd_major;             // 1: first-round items numbered XCD-major (see attn_kernel)
  int first_round;           // workgroups in the grid
  int tree_lds_half;         // LDS bytes for tree K (and again for tree V); multiple of 1 KiB
  int ns;                    // KV ring slots in LDS, 1..kMaxRingSlots
  int force_leave;           // test hook: odd chunks of first-round groups leave without waiting
  float scale_log2;          // softmax_scale * log2(e)
};

// Workspace layout for a given shape (host and device agree on it).
struct WsLayout {
  size_t arrive_off, partial_off, total;
  int rp_max, rows_slot, slot_floats, num_groups, s_max, chunk;
  int item_slots;
};

__host__ __device__ inline int cdiv(int a, int b) { return (a + b - 1) / b; }

// A batch whose longest prefix has `blocks` blocks, over `groups` groups,
// streams every sequence in one chunk.
__host__ __device__ inline bool one_chunk_batch(int blocks, long long groups) {
  return blocks <= kOneChunkBlocksBatch ||
         (blocks <= kOneChunkBlocksWide && groups >= kOneChunkWideGroups);
}

// Floats per chunk-partial slot: rows_slot fp32 o rows of D, then the running
// max m and sum l of every row.
__host__ __device__ inline int slot_floats_of(int rows_slot, int D) { return rows_slot * (D + 2); }

// combine_kernel's launch shape, computed alike by the host and the kernel:
// NSLOT row slots of D / 4 lanes per workgroup; QG row slots share one row
// (the fewest, a power of two, whose QMAX partial loads per lane cover the S
// chunks), so a workgroup takes NSLOT / QG rows and a group of R rows (at
// most kRowsPerPass) needs wpg workgroups.
template <int D>
__host__ __device__ inline int combine_qg(int S) {
  constexpr int QMAX = kMaxSplits / (kAttnThreads / (D / 4));
  int qg = 1;
  while (qg * QMAX < S) qg <<= 1;
  return qg;
}
template <int D>
__host__ __device__ inline int combine_wpg(int rows, int qg) {
  return cdiv(rows < kRowsPerPass ? rows : kRowsPerPass, kAttnThreads / (D / 4) / qg);
}
__host__ __device__ inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

}  // namespace ta
