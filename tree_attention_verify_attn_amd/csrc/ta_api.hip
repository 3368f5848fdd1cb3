// Host side of libtreeattn.so: argument checks, workspace layout, the work-item
// size heuristic, and kernel launches.  The C entry points are declared and
// documented in include/tree_attn.h.
#include <math.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>
#include <unordered_map>

#include "ta_kernels.hip"
#include "ta_commit.hip"
#include "tree_attn.h"

namespace ta {
namespace {

struct DeviceInfo {
  int cus = 0;
};

DeviceInfo device_info() {
  static std::mutex mu;
  static std::unordered_map<int, DeviceInfo> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return DeviceInfo{};
  std::lock_guard<std::mutex> lock(mu);
  auto it = cache.find(dev);
  if (it != cache.end()) return it->second;
  DeviceInfo d;
  if (hipDeviceGetAttribute(&d.cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    d.cus = 0;
  cache[dev] = d;
  return d;
}

// Resident workgroups per CU for a kernel and dynamic LDS size (cached).
int occupancy(const void* kernel, size_t dyn) {
  static std::mutex mu;
  static std::unordered_map<unsigned long long, int> cache;
  int dev = 0;
  (void)hipGetDevice(&dev);
  const unsigned long long key = (reinterpret_cast<unsigned long long>(kernel) << 8) ^
                                 (dyn << 1) ^ (static_cast<unsigned long long>(dev) << 40);
  std::lock_guard<std::mutex> lock(mu);
  auto it = cache.find(key);
  if (it != cache.end()) return it->second;
  // 0 when the launch does not fit a CU (too much LDS)
  int occ = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, kernel, kAttnThreads, dyn) != hipSuccess)
    occ = 1;
  if (occ < 0) occ = 0;
  cache[key] = occ;
  return occ;
}

// Raise a kernel's dynamic-LDS limit to at least `dyn` bytes.  The attribute
// is set once per kernel, device and size, not on every call, so that calls
// made while a stream is being captured into a graph make no runtime call
// beyond the launch itself (the first call of a shape, usually made outside
// any capture, sets it).
int ensure_dyn_lds(const void* kernel, size_t dyn) {
  static std::mutex mu;
  static std::unordered_map<unsigned long long, size_t> done;
  int dev = 0;
  (void)hipGetDevice(&dev);
  const unsigned long long key =
      reinterpret_cast<unsigned long long>(kernel) ^ (static_cast<unsigned long long>(dev) << 48);
  std::lock_guard<std::mutex> lock(mu);
  auto it = done.find(key);
  if (it != done.end() && it->second >= dyn) return kOk;
  if (hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, int(dyn)) != hipSuccess)
    return kErrHip;
  done[key] = dyn;
  return kOk;
}

// Test hook, read on every call: with TREE_ATTN_TEST_FORCE_LEAVE=1 in the
// environment, the odd chunks of every first-round group leave the meeting
// without waiting, as they do when the rest of their group has not started
// (the results must not change).  Never needed outside the tests.
int test_force_leave() {
  const char* v = getenv("TREE_ATTN_TEST_FORCE_LEAVE");
  return v && v[0] == '1' ? 1 : 0;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_shape(const ta_shape* s) {
  if (!s) return kErrInvalidArg;
  if (s->dtype != TA_DTYPE_F32 && s->dtype != TA_DTYPE_BF16) return kErrInvalidArg;
  if (s->batch < 1 || s->num_q_heads < 1 || s->num_kv_heads < 1) return kErrInvalidArg;
  if (s->num_q_heads % s->num_kv_heads != 0) return kErrInvalidArg;
  if (s->batch > kMaxBatch) return kErrUnsupported;
  if (s->head_dim != 64 && s->head_dim != 128) return kErrUnsupported;
  if (s->block_size != kBlock) return kErrUnsupported;
  if (s->max_blocks_per_seq < 1) return kErrInvalidArg;
  if (s->max_tree_nodes < 1) return kErrInvalidArg;
  if (s->max_tree_nodes > kMaxTreeSplit) return kErrUnsupported;
  if (s->max_prefix_len < 0) return kErrInvalidArg;
  if (static_cast<long long>(s->max_prefix_len) > static_cast<long long>(kBlock) * s->max_blocks_per_seq)
    return kErrInvalidArg;
  if (s->total_tree_nodes < 0) return kErrInvalidArg;
  if (s->num_blocks < 0 || (s->max_prefix_len > 0 && s->num_blocks < 1)) return kErrInvalidArg;
  if (s->split_tokens < 0 || s->split_tokens % kBlock != 0) return kErrInvalidArg;
  if (s->split_tokens > 4096) return kErrUnsupported;
  const long long groups = static_cast<long long>(s->batch) * s->num_kv_heads *
                           cdiv(s->max_tree_nodes * (s->num_q_heads / s->num_kv_heads), kRowsPerPass);
  if (groups > kMaxGroups) return kErrUnsupported;
  if (!(s->softmax_scale <= 0.f || isfinite(s->softmax_scale))) return kErrInvalidArg;
  return kOk;
}

int group_of(const ta_shape* s) { return s->num_q_heads / s->num_kv_heads; }

const void* attn_kernel_ptr(const ta_shape* s, bool fused);

// LDS bytes for the tree K rows (the same again for tree V) of the fused kernel.
// Trees of more than 64 nodes stage no rows there (their segments go through
// the ring); the area then holds the nodes' mask words and links instead.
int tree_lds_half(const ta_shape* s, bool fused) {
  if (!fused) return 0;
  if (s->max_tree_nodes > kMaxTree) {
    const int bytes = kMaxTreeSplit * (kMaxTreeSplit / 64) * 8 + kMaxTreeSplit * 4;
    return 1024 * cdiv(cdiv(bytes, 2), 1024);
  }
  const int rowb = s->head_dim * (s->dtype == TA_DTYPE_BF16 ? 2 : 4);
  return 1024 * cdiv(s->max_tree_nodes * rowb, 1024);
}

// Dynamic LDS of the attention kernel: tree rows, then the per-XCD item table.
// bytes of one KV ring slot (a 64-token K tile and V tile)
size_t ring_slot_bytes(const ta_shape* s) {
  return size_t(2) * kBlock * s->head_dim * (s->dtype == TA_DTYPE_BF16 ? 2 : 4);
}

// ints of the sequence table: cum[B + 1], ot[B], pl[B], perm[pow2 >= B]
size_t table_ints(const ta_shape* s) {
  size_t np = 1;
  while (np < size_t(s->batch)) np <<= 1;
  return size_t(3 * s->batch + 1) + np;
}

// LDS of the attention kernel besides the ring: tree rows, sequence table
// and the static SmemMisc
size_t attn_fixed_lds(const ta_shape* s, bool fused) {
  size_t bytes = 2 * size_t(tree_lds_half(s, fused));
  bytes += table_ints(s) * sizeof(int);
  return 16 * ((bytes + 15) / 16) + sizeof(SmemMisc) + 256;
}

// Ring slots that fit in one CU's LDS (0 if not even one does).
int ring_slots(const ta_shape* s, bool fused) {
  const size_t fixed = attn_fixed_lds(s, fused);
  if (fixed >= size_t(kLdsBytes)) return 0;
  size_t n = (size_t(kLdsBytes) - fixed) / ring_slot_bytes(s);
  return int(n < size_t(kMaxRingSlots) ? n : size_t(kMaxRingSlots));
}

size_t attn_dyn_lds(const ta_shape* s, bool fused) {
  size_t bytes = size_t(ring_slots(s, fused)) * ring_slot_bytes(s);
  bytes += 2 * size_t(tree_lds_half(s, fused));
  bytes += table_ints(s) * sizeof(int);
  return 16 * ((bytes + 15) / 16);
}

// Resident prefix-pass workgroups per XCD (bounds the splits of one group).
int grid_capacity(const ta_shape* s, bool fused) {
  int cus = device_info().cus;
  if (cus <= 0) cus = 256;  // no device: size for a full MI355X, one workgroup per CU
  const int occ = occupancy(attn_kernel_ptr(s, fused), attn_dyn_lds(s, fused));
  const int cap = cus * (occ > 0 ? occ : 1);
  return cap < kBarrierSlots ? cap : kBarrierSlots;
}

// One sequence whose tree is every row of q: items are numbered without a
// sequence table (and the chunk is the host's).
bool one_sequence(const ta_shape* s) {
  return s->batch == 1 && s->total_tree_nodes >= 1 && s->total_tree_nodes <= s->max_tree_nodes;
}

// Prefix tokens per work item.  Every XCD gets the groups (sequence, KV head,
// row pass) assigned to it; the chunk is sized so that each XCD has about one
// resident workgroup per work item, within [64, 4096] tokens.  A group never
// splits into more chunks than one XCD can hold resident at once (its items
// wait for each other) nor more than kMaxSplits.
int choose_chunk(const ta_shape* s, bool fused) {
  const int P = s->max_prefix_len > 0 ? s->max_prefix_len : 1;
  const int cap = grid_capacity(s, fused);
  const int max_splits = cap < kMaxSplits ? cap : kMaxSplits;
  const int min_chunk = kBlock * cdiv(cdiv(P, max_splits), kBlock);
  int chunk;
  const int nb = cdiv(P, kBlock);
  const int G = group_of(s);
  const long long groups = static_cast<long long>(s->batch) * s->num_kv_heads *
                           cdiv(s->max_tree_nodes * G, kRowsPerPass);
  if (s->split_tokens > 0) {
    chunk = s->split_tokens;
  } else if (one_sequence(s) ? nb <= kOneChunkBlocks : one_chunk_batch(nb, groups)) {
    chunk = nb * kBlock;  // short prefixes: one chunk, no exchange
  } else {
    // one sequence: fill about four fifths of the grid rather than all of it.
    // Fewer, longer chunks stream no slower (the CUs share the HBM) and
    // shrink the partial exchange: the 8k verify with 8 KV heads runs 208
    // items of 5 blocks faster than 256 items of 4.
    const long long fill = one_sequence(s) ? cap - cap / 5 : cap;
    const long long tok = (groups * P + fill - 1) / fill;
    chunk = static_cast<int>(kBlock * ((tok + kBlock - 1) / kBlock));
  }
  if (chunk < kBlock) chunk = kBlock;
  if (chunk > 4096) chunk = 4096;
  if (chunk < min_chunk) chunk = min_chunk;
  return chunk;
}

// The kernel picks the chunk from the actual prefix lengths unless the caller
// fixed it or the launch numbers items without a table.
bool chunk_auto(const ta_shape* s) {
  // (where the host's chunk is already one chunk per sequence, the launch
  // needs only a workgroup per group)
  const long long groups = static_cast<long long>(s->batch) * s->num_kv_heads *
                           cdiv(s->max_tree_nodes * group_of(s), kRowsPerPass);
  return s->split_tokens == 0 && !one_sequence(s) &&
         !one_chunk_batch(cdiv(s->max_prefix_len, kBlock), groups);
}

// Item slots a launch may use beyond groups x chunks-per-group: with the
// kernel's own chunk every item fits in the grid's first round.
int auto_cap(const ta_shape* s, bool fused) { return chunk_auto(s) ? grid_capacity(s, fused) : 0; }

WsLayout layout_for(const ta_shape* s, int chunk, int min_item_slots = 0) {
  WsLayout L{};
  const int G = group_of(s);
  const int D = s->head_dim;
  L.chunk = chunk;
  L.rp_max = cdiv(s->max_tree_nodes * G, kRowsPerPass);
  int rows = s->max_tree_nodes * G;
  if (rows > kRowsPerPass) rows = kRowsPerPass;
  L.rows_slot = 16 * cdiv(rows, 16);
  L.slot_floats = slot_floats_of(L.rows_slot, D);
  L.num_groups = s->batch * s->num_kv_heads * L.rp_max;
  L.s_max = s->max_prefix_len > 0 ? cdiv(s->max_prefix_len, chunk) : 1;
  // large batches: dense per-XCD numbering from a prefix table; small: static
  L.item_slots = L.num_groups * L.s_max;
  if (L.item_slots < min_item_slots) L.item_slots = min_item_slots;
  L.arrive_off = sizeof(WsHeader);
  // barrier pairs, then ticket counters (the kernel addresses both from the
  // region's start); neither depends on the shape
  L.partial_off = L.arrive_off + sizeof(unsigned) * (size_t(kCounterStride) * kBarrierSlots + kMaxGroups);
  static_assert(sizeof(WsHeader) % 256 == 0, "barrier region and partials stay 256-byte aligned");
  L.total = L.partial_off +
            size_t(L.item_slots) * L.slot_floats * sizeof(float);
  return L;
}

Params base_params(const ta_shape* s, const WsLayout& L, void* ws) {
  Params p{};
  p.batch = s->batch;
  p.hq = s->num_q_heads;
  p.hkv = s->num_kv_heads;
  p.group = group_of(s);
  p.head_dim = s->head_dim;
  p.max_blocks = s->max_blocks_per_seq;
  p.max_tree = s->max_tree_nodes;
  p.mask_words = cdiv(s->max_tree_nodes, 64);
  p.max_prefix = s->max_prefix_len;
  p.total_nodes = s->total_tree_nodes;
  p.num_blocks = s->num_blocks;
  p.chunk = L.chunk;
  p.rp_max = L.rp_max;
  p.rows_slot = L.rows_slot;
  p.slot_floats = L.slot_floats;
  p.num_groups = L.num_groups;
  p.s_max = L.s_max;
  p.item_slots = L.item_slots;
  // one sequence whose tree is every row of q: no sequence table needed
  p.single = one_sequence(s) ? 1 : 0;
  p.chunk_auto = chunk_auto(s) ? 1 : 0;
  p.single_items = p.single ? s->num_kv_heads * cdiv(s->total_tree_nodes * p.group, kRowsPerPass) * L.s_max : 0;
  const float scale = s->softmax_scale > 0.f ? s->softmax_scale : 1.f / sqrtf(float(s->head_dim));
  p.scale_log2 = scale * kLog2e;
  p.force_leave = test_force_leave();
  char* w = static_cast<char*>(ws);
  p.hdr = reinterpret_cast<WsHeader*>(w);
  if (w) {
    p.arrive = reinterpret_cast<unsigned*>(w + L.arrive_off);
    p.partials = reinterpret_cast<float*>(w + L.partial_off);
  }
  return p;
}

int launch_status() {
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? kOk : kErrHip;
}

// Fused launches for trees of more than kMaxTree nodes run their own kernel
// (the tree's segments through the ring), so that the common fused kernel
// keeps its registers.
bool big_fused(const ta_shape* s, bool fused) { return fused && s->max_tree_nodes > kMaxTree; }

// Instantiations that have the two-launch form.  The compiler's gfx950
// backend rejects the bf16, D = 64 large-tree attention kernel in that form
// (an illegal VOPC compare on src_shared_base), so that one combination meets
// in the launch whatever its chunk count.
template <typename T, int D, bool BIG>
constexpr bool two_launch_builds() { return !(sizeof(T) == 2 && D == 64 && BIG); }
bool two_launch_builds(const ta_shape* s, bool fused) {
  return !(s->dtype == TA_DTYPE_BF16 && s->head_dim == 64 && big_fused(s, fused));
}

template <typename T, int D, bool FUSED>
const void* attn_ptr(bool big, bool two = false) {
  if constexpr (FUSED)
    if (big) {
      if constexpr (two_launch_builds<T, D, true>())
        if (two) return reinterpret_cast<const void*>(&attn_kernel<T, D, true, true, true>);
      return reinterpret_cast<const void*>(&attn_kernel<T, D, true, true>);
    }
  return two ? reinterpret_cast<const void*>(&attn_kernel<T, D, FUSED, false, true>)
             : reinterpret_cast<const void*>(&attn_kernel<T, D, FUSED>);
}

const void* attn_kernel_ptr(const ta_shape* s, bool fused) {
  const bool big = big_fused(s, fused);
  if (s->dtype == TA_DTYPE_BF16) {
    if (s->head_dim == 128) return fused ? attn_ptr<uint16_t, 128, true>(big) : attn_ptr<uint16_t, 128, false>(big);
    return fused ? attn_ptr<uint16_t, 64, true>(big) : attn_ptr<uint16_t, 64, false>(big);
  }
  if (s->head_dim == 128) return fused ? attn_ptr<float, 128, true>(big) : attn_ptr<float, 128, false>(big);
  return fused ? attn_ptr<float, 64, true>(big) : attn_ptr<float, 64, false>(big);
}

// The split path's tree piece: one workgroup per (sequence, KV head, row
// pass), its dynamic LDS a ring of as many 64-node segments as fit.
template <typename T, int D>
int launch_suffix(const ta_shape* s, Params p, unsigned grid, hipStream_t stream) {
  const void* kern = reinterpret_cast<const void*>(&suffix_kernel<T, D>);
  const size_t slot = ring_slot_bytes(s);
  const size_t room = size_t(kLdsBytes) - sizeof(SmemMisc) - 256;
  int ns = int(room / slot);
  if (ns > kMaxRingSlots) ns = kMaxRingSlots;
  if (ns < 1) return kErrUnsupported;
  p.ns = ns;
  p.tree_lds_half = 0;
  const size_t dyn = size_t(ns) * slot;
  if (ensure_dyn_lds(kern, dyn) != kOk) return kErrHip;
  hipLaunchKernelGGL((suffix_kernel<T, D>), dim3(grid), dim3(kAttnThreads), dyn, stream, p);
  return launch_status();
}

// The second launch of a two-launch call (after attn_kernel on the same
// stream): QG row slots per row, the fewest whose QMAX partial loads per lane
// cover the S chunks; wpg workgroups per group.
template <typename T, int D, bool FUSED>
int launch_combine(const Params& p, hipStream_t stream) {
  const int st = launch_status();
  if (st != kOk) return st;
  constexpr int NSLOT = kAttnThreads / (D / 4);
  const int qg = combine_qg<D>(p.s_max);
  if (qg > NSLOT) return kErrUnsupported;  // more chunks than kMaxSplits (the chunk choice prevents it)
  const int rows = p.total_nodes * p.group;
  const int rp = cdiv(rows, kRowsPerPass);
  const int wpg = combine_wpg<D>(rows, qg);
  using OutT = typename std::conditional<FUSED, T, float>::type;
  // scalar arguments only: the first 14 dwords arrive preloaded in SGPRs
  hipLaunchKernelGGL((combine_kernel<OutT, D>), dim3(unsigned(p.hkv * rp * wpg)),
                     dim3(kAttnThreads), 0, stream, static_cast<const float*>(p.partials),
                     p.prefix_lens, static_cast<OutT*>(p.out), p.lse_out, p.s_max, p.group,
                     p.total_nodes, p.rows_slot, p.hq, p.max_prefix, p.chunk);
  return launch_status();
}

template <typename T, int D, bool FUSED>
int launch_attn(const ta_shape* s, Params p, const WsLayout& L, hipStream_t stream) {
  const bool big = big_fused(s, FUSED);
  const void* kern = attn_ptr<T, D, FUSED>(big);
  p.tree_lds_half = tree_lds_half(s, FUSED);
  p.ns = ring_slots(s, FUSED);
  if (p.ns < 1) return kErrUnsupported;  // tree rows + sequence table leave no room for the ring
  const size_t dyn = attn_dyn_lds(s, FUSED);
  if (ensure_dyn_lds(kern, dyn) != kOk) return kErrHip;
  const int cus = device_info().cus;
  if (cus <= 0) return kErrHip;
  const int occ = occupancy(kern, dyn);
  if (occ < 1) return kErrUnsupported;  // tree rows + item table exceed the LDS
  const int cap = cus * occ;
  int first = L.item_slots < cap ? L.item_slots : cap;
  if (first > kBarrierSlots) first = kBarrierSlots;  // one barrier pair per item of the first round
  if (first < 1) first = 1;
  p.first_round = first;
  // One-sequence launches number their items XCD-major: workgroup b, on XCD
  // b % 8 of the 8 that take workgroups in turn, gets item
  // (b % 8) * items / 8 + b / 8, so consecutive items share an XCD.
  //  - With several row passes every KV block is read once per row pass; the
  //    row passes of a KV head then run side by side on one XCD and stream
  //    the same blocks at the same time, so all but the first read hit that
  //    XCD's L2.
  //  - With one row pass the chunks of a KV head share an XCD (the 8 KV heads
  //    of a 32/8-head model fill the 8 XCDs); measured 0.3 us faster on the
  //    8k verify, though every exchange still goes through device-coherent
  //    memory.
  p.xcd_major = p.single && p.single_items % 8 == 0 && p.single_items <= first ? 1 : 0;
  // Two launches for a one-sequence launch whose groups have several chunks,
  // all in the first round: attn_kernel ends at the partial stores and
  // combine_kernel, queued behind it, folds them.  The kernel boundary costs
  // less than the chunks' meeting in the launch, and the attention kernel
  // without the meeting and combine code is leaner (measured on the 8k
  // verify: 16.2 us against 17.5 with 26 chunks a group, 12.6 against 14.8
  // with 64, 61.2 against 63.2 with 2).
  const bool two = p.single && p.single_items <= first && p.s_max >= kTwoLaunchMinChunks &&
                   two_launch_builds(s, FUSED);
  if (two) {
    if (ensure_dyn_lds(attn_ptr<T, D, FUSED>(big, true), dyn) != kOk) return kErrHip;
    if constexpr (FUSED && two_launch_builds<T, D, true>())
      if (big) {
        hipLaunchKernelGGL((attn_kernel<T, D, true, true, true>), dim3(unsigned(first)),
                           dim3(kAttnThreads), dyn, stream, p);
        return launch_combine<T, D, FUSED>(p, stream);
      }
    hipLaunchKernelGGL((attn_kernel<T, D, FUSED, false, true>), dim3(unsigned(first)),
                       dim3(kAttnThreads), dyn, stream, p);
    return launch_combine<T, D, FUSED>(p, stream);
  }
  if constexpr (FUSED)
    if (big) {
      hipLaunchKernelGGL((attn_kernel<T, D, true, true>), dim3(unsigned(first)), dim3(kAttnThreads),
                         dyn, stream, p);
      return launch_status();
    }
  hipLaunchKernelGGL((attn_kernel<T, D, FUSED>), dim3(unsigned(first)), dim3(kAttnThreads),
                     dyn, stream, p);
  return launch_status();
}

template <bool FUSED>
int dispatch_attn(const ta_shape* s, Params p, const WsLayout& L, hipStream_t stream) {
  if (s->dtype == TA_DTYPE_BF16) {
    if (s->head_dim == 128) return launch_attn<uint16_t, 128, FUSED>(s, p, L, stream);
    return launch_attn<uint16_t, 64, FUSED>(s, p, L, stream);
  }
  if (s->head_dim == 128) return launch_attn<float, 128, FUSED>(s, p, L, stream);
  return launch_attn<float, 64, FUSED>(s, p, L, stream);
}

int check_ws(const ta_shape* s, const WsLayout& L, void* ws, size_t ws_bytes) {
  (void)s;
  if (!ws || !aligned16(ws)) return kErrWorkspace;
  if (ws_bytes < L.total) return kErrWorkspace;
  return kOk;
}

// tree_attn_verify on a given workspace (argument checks, layout, launch).
int fused_verify(const ta_shape* shape, const void* q, const void* k_cache, const void* v_cache,
                 const int32_t* block_table, const int32_t* prefix_lens, const void* k_tree,
                 const void* v_tree, const int32_t* parents, const int32_t* tree_offsets,
                 void* out, float* lse_out, void* ws, size_t ws_bytes, hipStream_t stream) {
  int st = check_shape(shape);
  if (st != kOk) return st;
  if (!prefix_lens || !tree_offsets || !block_table) return kErrInvalidArg;
  if (shape->total_tree_nodes > 0 && (!q || !k_tree || !v_tree || !parents || !out))
    return kErrInvalidArg;
  if (shape->max_prefix_len > 0 && (!k_cache || !v_cache)) return kErrInvalidArg;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(k_tree) ||
      !aligned16(v_tree))
    return kErrInvalidArg;
  WsLayout L = layout_for(shape, choose_chunk(shape, true), auto_cap(shape, true));
  st = check_ws(shape, L, ws, ws_bytes);
  if (st != kOk) return st;
  if (shape->total_tree_nodes == 0) return kOk;
  Params p = base_params(shape, L, ws);
  p.q = q;
  p.k_cache = k_cache;
  p.v_cache = v_cache;
  p.block_table = block_table;
  p.prefix_lens = prefix_lens;
  p.k_tree = k_tree;
  p.v_tree = v_tree;
  p.parents = parents;
  p.tree_offsets = tree_offsets;
  p.out = out;
  p.lse_out = lse_out;
  return dispatch_attn<true>(shape, p, L, stream);
}

}  // namespace
}  // namespace ta

using namespace ta;

extern "C" {

size_t tree_attn_workspace_size(const ta_shape* shape) {
  if (check_shape(shape) != kOk) return 0;
  const size_t a = layout_for(shape, choose_chunk(shape, true), auto_cap(shape, true)).total;
  const size_t b = layout_for(shape, choose_chunk(shape, false), auto_cap(shape, false)).total;
  return a > b ? a : b;
}

int32_t tree_attn_split_tokens(const ta_shape* shape) {
  if (check_shape(shape) != kOk) return 0;
  return choose_chunk(shape, true);
}

ta_status tree_attn_launch_info(const ta_shape* shape, int32_t* info) {
  if (!info) return TA_ERR_INVALID_ARG;
  const int st = check_shape(shape);
  if (st != kOk) return static_cast<ta_status>(st);
  const int chunk = choose_chunk(shape, true);
  const WsLayout L = layout_for(shape, chunk, auto_cap(shape, true));
  const int cap = grid_capacity(shape, true);
  int grid = L.item_slots < cap ? L.item_slots : cap;
  if (grid < 1) grid = 1;
  int mode;
  if (one_sequence(shape))  // items numbered statically: the count is known here
    mode = L.item_slots > grid ? 1
           : L.s_max >= kTwoLaunchMinChunks && two_launch_builds(shape, true) ? 3 : 0;
  else if (chunk_auto(shape))
    mode = L.num_groups > grid ? 1 : 2;   // the kernel fits every item in the first round if it can
  else
    mode = L.item_slots <= grid ? 0 : 2;  // a fixed chunk: the actual prefix lengths decide
  info[0] = chunk;
  info[1] = grid;
  info[2] = L.item_slots;
  info[3] = mode;
  return TA_OK;
}

ta_status tree_attn_workspace_init(void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!ws || !aligned16(ws)) return TA_ERR_INVALID_ARG;
  if (ws_bytes == 0) return TA_OK;
  const size_t n16 = ws_bytes / 16;
  const size_t tail = ws_bytes % 16;
  size_t blocks = (n16 + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(ws_init_kernel, dim3(unsigned(blocks)), dim3(256), 0, stream,
                     static_cast<uint4*>(ws), n16, static_cast<char*>(ws) + n16 * 16, tail);
  return static_cast<ta_status>(launch_status());
}

ta_status tree_attn_build_mask(const ta_shape* shape, const int32_t* parents,
                               const int32_t* tree_offsets, uint64_t* mask_out, void* ws,
                               size_t ws_bytes, hipStream_t stream) {
  int st = check_shape(shape);
  if (st != kOk) return static_cast<ta_status>(st);
  if (!tree_offsets || !mask_out || (shape->total_tree_nodes > 0 && !parents))
    return TA_ERR_INVALID_ARG;
  if (!ws || !aligned16(ws) || ws_bytes < sizeof(WsHeader)) return TA_ERR_WORKSPACE;
  WsLayout L = layout_for(shape, kBlock);
  Params p = base_params(shape, L, ws);
  p.parents = parents;
  p.tree_offsets = tree_offsets;
  if (p.mask_words == 1)
    hipLaunchKernelGGL(mask_kernel, dim3(unsigned(shape->batch)), dim3(64), 0, stream, p, mask_out);
  else
    hipLaunchKernelGGL(mask_words_kernel, dim3(unsigned(shape->batch)), dim3(kMaxTreeSplit), 0,
                       stream, p, mask_out);
  return static_cast<ta_status>(launch_status());
}

ta_status tree_attn_prefix(const ta_shape* shape, const void* q, const void* k_cache,
                           const void* v_cache, const int32_t* block_table,
                           const int32_t* prefix_lens, const int32_t* tree_offsets,
                           float* o_prefix, float* lse_prefix, void* ws, size_t ws_bytes,
                           hipStream_t stream) {
  int st = check_shape(shape);
  if (st != kOk) return static_cast<ta_status>(st);
  if (!prefix_lens || !tree_offsets || !lse_prefix || !block_table) return TA_ERR_INVALID_ARG;
  if (shape->total_tree_nodes > 0 && (!q || !o_prefix)) return TA_ERR_INVALID_ARG;
  if (shape->max_prefix_len > 0 && (!k_cache || !v_cache)) return TA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(o_prefix))
    return TA_ERR_INVALID_ARG;
  WsLayout L = layout_for(shape, choose_chunk(shape, false), auto_cap(shape, false));
  st = check_ws(shape, L, ws, ws_bytes);
  if (st != kOk) return static_cast<ta_status>(st);
  if (shape->total_tree_nodes == 0) return TA_OK;
  Params p = base_params(shape, L, ws);
  p.q = q;
  p.k_cache = k_cache;
  p.v_cache = v_cache;
  p.block_table = block_table;
  p.prefix_lens = prefix_lens;
  p.tree_offsets = tree_offsets;
  p.out = o_prefix;
  p.lse_out = lse_prefix;
  return static_cast<ta_status>(dispatch_attn<false>(shape, p, L, stream));
}

ta_status tree_attn_suffix(const ta_shape* shape, const void* q, const void* k_tree,
                           const void* v_tree, const uint64_t* mask,
                           const int32_t* tree_offsets, float* o_suffix, float* lse_suffix,
                           hipStream_t stream) {
  int st = check_shape(shape);
  if (st != kOk) return static_cast<ta_status>(st);
  if (!tree_offsets || !lse_suffix) return TA_ERR_INVALID_ARG;
  if (shape->total_tree_nodes > 0 && (!q || !k_tree || !v_tree || !mask || !o_suffix))
    return TA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k_tree) || !aligned16(v_tree) || !aligned16(o_suffix))
    return TA_ERR_INVALID_ARG;
  if (shape->total_tree_nodes == 0) return TA_OK;
  WsLayout L = layout_for(shape, kBlock);
  Params p = base_params(shape, L, nullptr);
  p.q = q;
  p.k_tree = k_tree;
  p.v_tree = v_tree;
  p.mask_in = mask;
  p.tree_offsets = tree_offsets;
  p.out = o_suffix;
  p.lse_out = lse_suffix;
  const unsigned grid = unsigned(L.num_groups);
  if (shape->dtype == TA_DTYPE_BF16)
    st = shape->head_dim == 128 ? launch_suffix<uint16_t, 128>(shape, p, grid, stream)
                                : launch_suffix<uint16_t, 64>(shape, p, grid, stream);
  else
    st = shape->head_dim == 128 ? launch_suffix<float, 128>(shape, p, grid, stream)
                                : launch_suffix<float, 64>(shape, p, grid, stream);
  return static_cast<ta_status>(st);
}

ta_status tree_attn_merge(int64_t rows, int32_t head_dim, ta_dtype out_dtype, const float* o_a,
                          const float* lse_a, const float* o_b, const float* lse_b, void* out,
                          float* lse_out, hipStream_t stream) {
  if (rows < 0 || head_dim < 4 || head_dim % 4 != 0) return TA_ERR_INVALID_ARG;
  if (out_dtype != TA_DTYPE_F32 && out_dtype != TA_DTYPE_BF16) return TA_ERR_INVALID_ARG;
  if (rows == 0) return TA_OK;
  if (!o_a || !lse_a || !o_b || !lse_b || !out) return TA_ERR_INVALID_ARG;
  if (!aligned16(o_a) || !aligned16(o_b)) return TA_ERR_INVALID_ARG;
  const long long n = rows * (head_dim / 4);
  long long blocks = (n + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  if (out_dtype == TA_DTYPE_BF16)
    hipLaunchKernelGGL((merge_kernel<uint16_t>), dim3(unsigned(blocks)), dim3(256), 0, stream,
                       static_cast<long long>(rows), int(head_dim), o_a, lse_a, o_b, lse_b,
                       static_cast<uint16_t*>(out), lse_out);
  else
    hipLaunchKernelGGL((merge_kernel<float>), dim3(unsigned(blocks)), dim3(256), 0, stream,
                       static_cast<long long>(rows), int(head_dim), o_a, lse_a, o_b, lse_b,
                       static_cast<float*>(out), lse_out);
  return static_cast<ta_status>(launch_status());
}

ta_status tree_attn_verify(const ta_shape* shape, const void* q, const void* k_cache,
                           const void* v_cache, const int32_t* block_table,
                           const int32_t* prefix_lens, const void* k_tree, const void* v_tree,
                           const int32_t* parents, const int32_t* tree_offsets, void* out,
                           float* lse_out, void* ws, size_t ws_bytes, hipStream_t stream) {
  return static_cast<ta_status>(fused_verify(shape, q, k_cache, v_cache, block_table, prefix_lens,
                                             k_tree, v_tree, parents, tree_offsets, out, lse_out,
                                             ws, ws_bytes, stream));
}

ta_status tree_attn_verify_incache(const ta_shape* shape, const void* q, const void* k_cache,
                                   const void* v_cache, const int32_t* block_table,
                                   const int32_t* prefix_lens, const int32_t* parents,
                                   const int32_t* tree_offsets, void* out, float* lse_out,
                                   void* ws, size_t ws_bytes, hipStream_t stream) {
  int st = check_shape(shape);
  if (st != kOk) return static_cast<ta_status>(st);
  if (!prefix_lens || !tree_offsets || !block_table || !k_cache || !v_cache)
    return TA_ERR_INVALID_ARG;
  if (shape->num_blocks < 1) return TA_ERR_INVALID_ARG;
  if (shape->total_tree_nodes > 0 && (!q || !parents || !out)) return TA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache)) return TA_ERR_INVALID_ARG;
  WsLayout L = layout_for(shape, choose_chunk(shape, true), auto_cap(shape, true));
  st = check_ws(shape, L, ws, ws_bytes);
  if (st != kOk) return static_cast<ta_status>(st);
  if (shape->total_tree_nodes == 0) return TA_OK;
  Params p = base_params(shape, L, ws);
  // one-sequence numbering needs spare lanes in the block-id load for the tree
  // region's blocks (the region's position is known only with P)
  if (L.chunk / kBlock + cdiv(shape->max_tree_nodes, kBlock) + 1 > 64) p.single = 0;
  p.tree_in_cache = 1;
  p.q = q;
  p.k_cache = k_cache;
  p.v_cache = v_cache;
  p.block_table = block_table;
  p.prefix_lens = prefix_lens;
  p.parents = parents;
  p.tree_offsets = tree_offsets;
  p.out = out;
  p.lse_out = lse_out;
  return static_cast<ta_status>(dispatch_attn<true>(shape, p, L, stream));
}

ta_status tree_attn_commit_incache(const ta_shape* shape, const int32_t* parents,
                                   const int32_t* tree_offsets, const int32_t* accept_len,
                                   const int32_t* accept_path, void* k_cache, void* v_cache,
                                   const int32_t* block_table, int32_t* prefix_lens, void* ws,
                                   size_t ws_bytes, hipStream_t stream) {
  int st = check_shape(shape);
  if (st != kOk) return static_cast<ta_status>(st);
  if (!tree_offsets || !accept_len || !accept_path || !block_table || !prefix_lens ||
      !k_cache || !v_cache)
    return TA_ERR_INVALID_ARG;
  if (shape->total_tree_nodes > 0 && !parents) return TA_ERR_INVALID_ARG;
  if (shape->num_blocks < 1 || !aligned16(k_cache) || !aligned16(v_cache)) return TA_ERR_INVALID_ARG;
  if (!ws || !aligned16(ws) || ws_bytes < sizeof(WsHeader)) return TA_ERR_WORKSPACE;
  IncacheParams c{};
  c.parents = parents;
  c.tree_offsets = tree_offsets;
  c.accept_len = accept_len;
  c.path = accept_path;
  c.k_cache = k_cache;
  c.v_cache = v_cache;
  c.block_table = block_table;
  c.prefix_lens = prefix_lens;
  c.hdr = static_cast<WsHeader*>(ws);
  c.batch = shape->batch;
  c.total_nodes = shape->total_tree_nodes;
  c.max_tree = shape->max_tree_nodes;
  c.max_blocks = shape->max_blocks_per_seq;
  c.num_blocks = shape->num_blocks;
  c.hkv = shape->num_kv_heads;
  c.row_bytes = shape->head_dim * (shape->dtype == TA_DTYPE_BF16 ? 2 : 4);
  hipLaunchKernelGGL(commit_incache_kernel, dim3(unsigned(shape->batch)), dim3(kThreads), 0,
                     stream, c);
  return static_cast<ta_status>(launch_status());
}

ta_status tree_attn_accept_greedy(const ta_shape* shape, const int32_t* parents,
                                  const int32_t* tree_offsets, const int32_t* draft_tokens,
                                  const int32_t* target_argmax, int32_t* accept_len,
                                  int32_t* accept_path, int32_t* bonus_token, void* ws,
                                  size_t ws_bytes, hipStream_t stream) {
  int st = check_shape(shape);
  if (st != kOk) return static_cast<ta_status>(st);
  if (!tree_offsets || !accept_len || !accept_path || !bonus_token) return TA_ERR_INVALID_ARG;
  if (shape->total_tree_nodes > 0 && (!parents || !draft_tokens || !target_argmax))
    return TA_ERR_INVALID_ARG;
  if (!ws || !aligned16(ws) || ws_bytes < sizeof(WsHeader)) return TA_ERR_WORKSPACE;
  AcceptParams a{};
  a.parents = parents;
  a.tree_offsets = tree_offsets;
  a.draft = draft_tokens;
  a.argmax = target_argmax;
  a.accept_len = accept_len;
  a.path = accept_path;
  a.bonus = bonus_token;
  a.hdr = static_cast<WsHeader*>(ws);
  a.batch = shape->batch;
  a.total_nodes = shape->total_tree_nodes;
  a.max_tree = shape->max_tree_nodes;
  if (shape->max_tree_nodes <= kMaxTree)
    hipLaunchKernelGGL(accept_kernel, dim3(unsigned(cdiv(shape->batch, kAcceptWaves))),
                       dim3(64 * kAcceptWaves), 0, stream, a);
  else  // multi-word ancestor sets: one 256-thread workgroup per tree
    hipLaunchKernelGGL(accept_words_kernel, dim3(unsigned(shape->batch)), dim3(kMaxTreeSplit), 0,
                       stream, a);
  return static_cast<ta_status>(launch_status());
}

ta_status tree_attn_commit(const ta_shape* shape, const void* k_tree, const void* v_tree,
                           const int32_t* parents, const int32_t* tree_offsets,
                           const int32_t* accept_len, const int32_t* accept_path,
                           void* k_cache, void* v_cache, int32_t* block_table,
                           int32_t* prefix_lens, const int32_t* free_blocks, int32_t free_count,
                           int32_t* blocks_taken, void* ws, size_t ws_bytes,
                           hipStream_t stream) {
  int st = check_shape(shape);
  if (st != kOk) return static_cast<ta_status>(st);
  if (!tree_offsets || !accept_len || !accept_path || !block_table || !prefix_lens)
    return TA_ERR_INVALID_ARG;
  if (shape->total_tree_nodes > 0 && (!parents || !k_tree || !v_tree)) return TA_ERR_INVALID_ARG;
  if (!k_cache || !v_cache || shape->num_blocks < 1) return TA_ERR_INVALID_ARG;
  if (free_count < 0 || (free_count > 0 && !free_blocks)) return TA_ERR_INVALID_ARG;
  if (!aligned16(k_tree) || !aligned16(v_tree) || !aligned16(k_cache) || !aligned16(v_cache))
    return TA_ERR_INVALID_ARG;
  if (!ws || !aligned16(ws)) return TA_ERR_WORKSPACE;
  const WsLayout L = layout_for(shape, kBlock);
  const size_t plan_bytes = sizeof(CommitPlan) * size_t(shape->batch);
  if (ws_bytes < L.partial_off + plan_bytes) return TA_ERR_WORKSPACE;
  char* w = static_cast<char*>(ws);
  CommitParams c{};
  c.k_tree = k_tree;
  c.v_tree = v_tree;
  c.parents = parents;
  c.tree_offsets = tree_offsets;
  c.accept_len = accept_len;
  c.path = accept_path;
  c.k_cache = k_cache;
  c.v_cache = v_cache;
  c.block_table = block_table;
  c.prefix_lens = prefix_lens;
  c.free_blocks = free_blocks;
  c.blocks_taken = blocks_taken;
  c.hdr = reinterpret_cast<WsHeader*>(w);
  c.plan = reinterpret_cast<CommitPlan*>(w + L.partial_off);
  c.batch = shape->batch;
  c.total_nodes = shape->total_tree_nodes;
  c.max_tree = shape->max_tree_nodes;
  c.max_blocks = shape->max_blocks_per_seq;
  c.num_blocks = shape->num_blocks;
  c.hkv = shape->num_kv_heads;
  c.row_bytes = shape->head_dim * (shape->dtype == TA_DTYPE_BF16 ? 2 : 4);
  c.free_count = free_count;
  hipLaunchKernelGGL(commit_check_kernel, dim3(unsigned(cdiv(shape->batch, kAcceptWaves))),
                     dim3(64 * kAcceptWaves), 0, stream, c);
  hipLaunchKernelGGL(commit_apply_kernel, dim3(unsigned(shape->batch)), dim3(kThreads), 0, stream, c);
  return static_cast<ta_status>(launch_status());
}

ta_status tree_attn_get_error(void* ws, hipStream_t stream) {
  if (!ws) return TA_ERR_INVALID_ARG;
  int err = 0;
  if (hipMemcpyAsync(&err, ws, sizeof(int), hipMemcpyDeviceToHost, stream) != hipSuccess)
    return TA_ERR_HIP;
  if (hipStreamSynchronize(stream) != hipSuccess) return TA_ERR_HIP;
  if (err != 0) {
    const int zero = 0;
    if (hipMemcpyAsync(ws, &zero, sizeof(int), hipMemcpyHostToDevice, stream) != hipSuccess)
      return TA_ERR_HIP;
    if (hipStreamSynchronize(stream) != hipSuccess) return TA_ERR_HIP;
  }
  return static_cast<ta_status>(err);
}

const char* tree_attn_status_string(ta_status status) {
  switch (status) {
    case TA_OK: return "ok";
    case TA_ERR_INVALID_ARG: return "invalid argument (scalar, null or misaligned pointer)";
    case TA_ERR_UNSUPPORTED: return "unsupported shape";
    case TA_ERR_BAD_TREE: return "invalid tree: parent array or tree_offsets (device check)";
    case TA_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
    case TA_ERR_HIP: return "HIP runtime error or kernel launch failure";
    case TA_ERR_BAD_PREFIX: return "prefix length or KV block id out of range (device check)";
    case TA_ERR_TIMEOUT: return "a bounded cross-workgroup wait gave up (device check)";
    case TA_ERR_NO_BLOCKS: return "free list or block-table row too small for the commit (device check)";
    case TA_ERR_SCRATCH: return "shape needs more workspace than the no-allocation entry point's static scratch";
  }
  return "unknown status";
}

}  // extern "C"

#include "ta_noalloc.hip"
