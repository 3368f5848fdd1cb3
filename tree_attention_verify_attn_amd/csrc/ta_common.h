// Definitions shared by the host entry points and the gfx950 kernels of the
// split tree-verify attention library.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace ta {

constexpr int kBlock = 64;        // tokens per KV-cache block
constexpr int kThreads = 256;     // threads per workgroup (4 wave64)
constexpr int kWaves = kThreads / 64;
constexpr int kMaxTree = 64;      // one 64-bit mask word per tree node
constexpr int kMaxBatch = 4096;   // per-workgroup item table lives in LDS
constexpr int kRowsPerPass = 64;  // grouped query rows one work item covers
constexpr int kMaxSplits = 64;    // cap on work items per (sequence, head, row pass)
constexpr unsigned kSpinLimit = 1u << 22;
constexpr int kMaxXcd = 16;       // XCDs per device the work numbering supports
constexpr int kCusPerXcd = 32;    // gfx950

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
  kErrPlacement = 8,
};

// First 256 bytes of every workspace.
struct WsHeader {
  int error;          // first device-detected error code (0 = none)
  unsigned done;      // workgroups that have left the persistent loop
  unsigned ticket[kMaxXcd];  // per-XCD next dynamically assigned work item
  unsigned pad[64 - 2 - kMaxXcd];
};
static_assert(sizeof(WsHeader) == 256, "workspace header is 256 bytes");

// Everything a kernel needs for one call.  Built on the host, passed by value.
//
// Work decomposition of the prefix pass.  A group is (sequence b, KV head g,
// row pass rp); its prefix is cut into chunks of `chunk` tokens, one work item
// each.  Workgroup i runs on XCD i % n_xcd (the hardware hands workgroups to
// the XCDs round robin), and every item of a group is given to workgroups of
// one XCD, so the group's partial results meet in that XCD's L2.  Items of XCD
// x are numbered li = 0, 1, ...; the first round takes li = i / n_xcd, later
// ones come from the XCD's ticket counter.
//   static numbering (table_mode 0): group k = lg * n_xcd + x, li = lg * s_max + s;
//   table numbering (table_mode 1): sequences b = x, x + n_xcd, ... live on XCD x
//     and their items are numbered densely from a per-workgroup prefix table.
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
  unsigned* arrive;          // per group arrival counters
  float* partials;           // [n_xcd * items_per_xcd][slot_floats]
  int batch, hq, hkv, group, head_dim;
  int max_blocks, max_tree, max_prefix, total_nodes, num_blocks;
  int chunk;                 // prefix tokens per work item (multiple of 64)
  int rp_max;                // row passes per (sequence, head)
  int rows_slot;             // rows reserved per partial slot
  int slot_floats;           // floats per partial slot
  int num_groups;            // batch * hkv * rp_max
  int n_xcd;                 // XCDs the grid spreads over
  int table_mode;            // 0 static numbering, 1 per-XCD sequence table
  int s_max;                 // chunks per group, upper bound
  int lg_per_xcd;            // static numbering: groups per XCD
  int seq_per_xcd;           // table numbering: sequences per XCD (upper bound)
  int items_per_xcd;         // item slots per XCD
  int first_round;           // workgroups per XCD in the grid
  int tree_lds_half;         // LDS bytes for tree K (and again for tree V); multiple of 1 KiB
  float scale_log2;          // softmax_scale * log2(e)
};

// Workspace layout for a given shape (host and device agree on it).
struct WsLayout {
  size_t arrive_off, partial_off, total;
  int rp_max, rows_slot, slot_floats, num_groups, s_max, chunk;
  int n_xcd, table_mode, lg_per_xcd, seq_per_xcd, items_per_xcd;
};

__host__ __device__ inline int cdiv(int a, int b) { return (a + b - 1) / b; }
__host__ __device__ inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

}  // namespace ta
