// gfx950 kernels of the split tree-verify attention library.
//
// Method: each draft-tree query attends to (a) its sequence's committed prefix,
// read through a paged KV cache, with no mask, and (b) the tree tokens on its
// root path.  The two partial results are combined exactly through their
// log-sum-exp.  [pith.science review of arXiv 2508.08192, "What carries the
// argument"; merge over disjoint KV chunks: Hydragen, Juravsky et al. 2024,
// pith.science verdict record, pith_extraction.supporting_citations; paged KV:
// PagedAttention, Kwon et al. 2023, same field]
//
// Kernels
//   ws_init_kernel   zero-fill of a workspace (graph-capture safe)
//   mask_kernel      ancestor-or-self mask words of every tree (one wave per tree)
//   attn_kernel      prefix pass; with FUSED it also builds the tree mask, runs
//                    the tree piece and merges (the fused verify)
//   combine_kernel   the split reduce of a one-sequence launch in two launches:
//                    folds the chunk partials of every group into its rows
//   suffix_kernel    tree piece on its own (split path), on the same MFMA path
//   merge_kernel     merge of two (o, lse) results (split path)
//
// attn_kernel, one work item = sequence b, KV head g, row pass rp, prefix chunk s,
// one workgroup of 8 waves per CU:
//   * the grouped query rows of (b, g) -- tree node i times the G query heads
//     sharing KV head g -- form up to four 16-row MFMA tiles;  wave w takes
//     row tile w % 4 and key half w / 4 of every 64-key block, with its own
//     online-softmax state (the two halves are merged once per item);
//   * the chunk's 64-token KV blocks go HBM -> LDS by direct DMA into a ring of
//     NS slots (K and V row-major with an XOR chunk swizzle), NS - 1 blocks
//     ahead of the one being consumed;
//   * per block each wave computes S^T = K Q^T (v_mfma_f32_16x16x32_bf16), so a
//     lane holds one query row and the online softmax needs only the cross-lane
//     steps l^16, l^32; V^T comes from the transposing LDS read and P^T feeds
//     O^T += V^T P^T as the MFMA B operand straight from registers;
//   * fused: the last chunk of a group also stages the group's tree rows and
//     runs them as one more 64-key block under the ancestor-or-self mask;
//   * a group with one chunk writes its output rows directly; otherwise each
//     chunk writes its partial (unnormalised o, running max, running sum) with
//     device-coherent stores, the chunks meet at a sense-reversing barrier and
//     split the final combine: each takes some rows, folds every chunk partial
//     with its log-sum-exp weight and writes the output rows.
//     A one-sequence launch whose groups have several chunks (the 8k-context
//     verify) instead ends at the partial stores; combine_kernel, queued right
//     after it on the same stream, does the combine.
#include <type_traits>

#include "ta_device.h"

namespace ta {

// Wait until every memory operation this wave issued has completed.
__device__ __forceinline__ void wait_all_mem() { __builtin_amdgcn_s_waitcnt(0); }

__device__ __forceinline__ unsigned ld_counter(const unsigned* p) {
  return __hip_atomic_load(const_cast<unsigned*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}


// =============================================================== utilities
__global__ void __launch_bounds__(256) ws_init_kernel(uint4* ws, size_t n16, char* tail,
                                                     size_t ntail) {
  const size_t stride = size_t(gridDim.x) * blockDim.x;
  for (size_t i = size_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n16; i += stride)
    ws[i] = make_uint4(0, 0, 0, 0);
  if (blockIdx.x == 0 && threadIdx.x < ntail) tail[threadIdx.x] = 0;
}

// Per-sequence facts, validated.  Invalid data is replaced by an empty tree or
// an empty prefix so that no later read goes out of bounds.
struct SeqInfo {
  int off, T, P, S, RP, items;
};

__device__ __forceinline__ SeqInfo make_seq(const Params& p, int o0, int o1, int P, bool flag) {
  SeqInfo s;
  int T = o1 - o0;
  const bool tree_ok = o0 >= 0 && o1 >= o0 && o1 <= p.total_nodes && T <= p.max_tree;
  const bool p_ok = P >= 0 && P <= p.max_prefix;
  if (!tree_ok) {
    if (flag) set_error(p.hdr, kErrBadTree);
    T = 0;
    o0 = 0;
  }
  if (!p_ok) {
    if (flag) set_error(p.hdr, kErrBadPrefix);
    P = 0;
  }
  s.off = o0;
  s.T = T;
  s.P = P;
  s.S = P > 0 ? cdiv(P, p.chunk) : 1;
  s.RP = cdiv(T * p.group, kRowsPerPass);
  s.items = p.hkv * s.RP * s.S;
  return s;
}

__device__ __forceinline__ SeqInfo seq_info(const Params& p, int b, bool flag) {
  return make_seq(p, p.tree_offsets[b], p.tree_offsets[b + 1], p.prefix_lens[b], flag);
}

// Per-workgroup sequence table in LDS, built once per launch.  Sequences are
// placed in processing order: when the items need more than one round of
// workgroups, longest prefix first (sorted by the class floor(log2 P),
// ties by index, the same order in every workgroup), so that the last items
// handed out are the shortest; otherwise in index order.  For position k:
// perm[k] = the sequence (low 11 bits), cum[k] = items before it, ot[k] =
// tree offset | tree size << 24, pl[k] = prefix length, all validated (the
// first workgroup flags bad data).  With it an item's facts need no global
// read.  Returns the item count.
constexpr int kTreeSizeShift = 23;  // tree offsets < 2^23 (<= 2048 trees of <= 256 nodes)
constexpr int kSeqBits = 11;        // sequence index bits in a sort key (batch <= 2048)
// Exclusive prefix sum of v over the workgroup's threads (in thread order) and
// the total: a scan inside each wave, then the wave totals through LDS (one
// barrier).  Every thread must call it.
__device__ __forceinline__ int block_exclusive_scan(int v, int* scratch, int& total) {
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int inc = wave_inclusive_sum(v);
  if (lane == 63) scratch[w] = inc;
  __syncthreads();
  int before = 0;
  total = 0;
#pragma unroll
  for (int x = 0; x < kAttnWaves; ++x) {
    const int t = scratch[x];
    before += x < w ? t : 0;
    total += t;
  }
  __syncthreads();  // scratch may be reused right after
  return before + inc - v;
}

// Sums of a and b and the max of c over the workgroup's threads; every
// thread must call it.  Two barriers.
__device__ __forceinline__ void block_sum2_max(int& a, int& b, int& c, int* scratch) {
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  a = wave_sum(a);
  b = wave_sum(b);
  c = wave_max(c);
  if (lane == 0) {
    scratch[w] = a;
    scratch[kAttnWaves + w] = b;
    scratch[2 * kAttnWaves + w] = c;
  }
  __syncthreads();
  a = b = c = 0;
#pragma unroll
  for (int x = 0; x < kAttnWaves; ++x) {
    a += scratch[x];
    b += scratch[kAttnWaves + x];
    c = max(c, scratch[2 * kAttnWaves + x]);
  }
  __syncthreads();
}

// Ascending bitonic sort of np keys (np a power of two, np <= kMaxBatch);
// element i = q * kAttnThreads + thread lives in keys[q] of that thread.
// Partners less than a wave apart meet by lane shuffles, partners in other
// waves through two LDS buffers in turn (xbuf: 2 * kMaxBatch ints, one
// barrier per such step), partners in another slot of the same thread in
// registers.  Every thread must call it.
constexpr int kSortSlots = kMaxBatch / kAttnThreads;
__device__ void bitonic_sort(int (&keys)[kSortSlots], int np, int* xbuf) {
  const int tid = threadIdx.x;
  int b = 0;
  for (int k = 2; k <= np; k <<= 1)
    for (int jj = k >> 1; jj > 0; jj >>= 1) {
      if (jj >= kAttnThreads) {
        const int qd = jj / kAttnThreads;
#pragma unroll
        for (int q = 0; q < kSortSlots; ++q) {
          const int qp = q ^ qd;
          if (qp > q && qp < kSortSlots) {
            const bool up = ((q * kAttnThreads + tid) & k) == 0;
            const int lo = min(keys[q], keys[qp]), hi = max(keys[q], keys[qp]);
            keys[q] = up ? lo : hi;
            keys[qp] = up ? hi : lo;
          }
        }
      } else {
        int other[kSortSlots];
        if (jj >= 64) {
          int* xb = xbuf + b * kMaxBatch;
#pragma unroll
          for (int q = 0; q < kSortSlots; ++q) xb[q * kAttnThreads + tid] = keys[q];
          __syncthreads();
#pragma unroll
          for (int q = 0; q < kSortSlots; ++q) other[q] = xb[q * kAttnThreads + (tid ^ jj)];
          b ^= 1;  // the next exchange writes the other buffer, so no second barrier
        } else {
#pragma unroll
          for (int q = 0; q < kSortSlots; ++q) other[q] = __shfl_xor(keys[q], jj);
        }
#pragma unroll
        for (int q = 0; q < kSortSlots; ++q) {
          const int i = q * kAttnThreads + tid;
          const bool keep_min = ((i & k) == 0) == ((i & jj) == 0);
          keys[q] = keep_min ? min(keys[q], other[q]) : max(keys[q], other[q]);
        }
      }
    }
}

// When the host leaves the chunk to the kernel (p.chunk_auto), the chunk
// comes from the actual prefix lengths.  If the longest is short enough
// (one_chunk_batch: up to 6 blocks, or 8 with 32 groups or more), every
// sequence streams in one chunk (its chunks would cost more to meet than to
// stream); otherwise, if the groups
// (sequence, KV head, row pass) are fewer than the grid's workgroups, the
// chunk is the smallest multiple of 64 tokens with which every item fits in
// the first round (the sum of the groups' chunk counts stays within the
// grid) and no group has more than kMaxSplits chunks.  `chunk` returns the
// chunk in force.
__device__ int build_table(const Params& p, int* cum, int* ot, int* pl, int* perm, int* scratch,
                           int* xbuf, int& chunk) {
  const int tid = threadIdx.x;
  const int n = p.batch;
  const int per = cdiv(n, kAttnThreads);
  const int j0 = min(n, tid * per);
  const int j1 = min(n, j0 + per);
  const bool flag = blockIdx.x == 0;
  // facts in index order, the item prefix in index order
  constexpr int kPerMax = kMaxBatch / kAttnThreads;
  int items_q[kPerMax], groups_q[kPerMax], p_q[kPerMax];
  int work = 0, groups = 0, max_blocks = 0;
#pragma unroll
  for (int q = 0; q < kPerMax; ++q) {
    const int j = j0 + q;
    groups_q[q] = 0;
    p_q[q] = 0;
    if (j < j1) {
      const SeqInfo si = seq_info(p, j, flag);
      ot[j] = int(unsigned(si.off) | (unsigned(si.T) << kTreeSizeShift));
      pl[j] = si.P;
      perm[j] = j;
      groups_q[q] = p.hkv * si.RP;
      p_q[q] = si.P;
      const int nb = cdiv(si.P, kBlock);
      work += groups_q[q] * nb;
      groups += groups_q[q];
      max_blocks = max(max_blocks, nb);
    }
  }
  chunk = p.chunk;
  if (p.chunk_auto) {
    block_sum2_max(work, groups, max_blocks, scratch);
    if (one_chunk_batch(max_blocks, groups)) {
      chunk = max(max_blocks, 1) * kBlock;  // short prefixes: one chunk each, no exchange
    } else if (groups < p.first_round) {
      int cb = max(cdiv(work, p.first_round - groups), cdiv(max_blocks, kMaxSplits));
      cb = min(max(cb, 1), kMaxChunk / kBlock);
      chunk = cb * kBlock;
    }
  }
  int local = 0;
#pragma unroll
  for (int q = 0; q < kPerMax; ++q) {
    items_q[q] = groups_q[q] * (p_q[q] > 0 ? cdiv(p_q[q], chunk) : 1);
    local += items_q[q];
  }
  int total = 0;
  int run = block_exclusive_scan(local, scratch, total);
  const bool sort = n > 1 && total > p.first_round;
  if (!sort) {
#pragma unroll
    for (int q = 0; q < kPerMax; ++q)
      if (j0 + q < j1) {
        cum[j0 + q] = run;
        run += items_q[q];
      }
  } else {
    // processing order: keys (length class, index) ascending = longest first
    const int np = [&] { int v = 1; while (v < n) v <<= 1; return v; }();
    __syncthreads();  // pl[] of every sequence is in LDS
    int keys[kSortSlots];
#pragma unroll
    for (int q = 0; q < kSortSlots; ++q) {
      const int i = q * kAttnThreads + tid;
      keys[q] = 0x7fffffff;  // padding sorts last
      if (i < n) {
        const int P = pl[i];
        const int cls = 31 - __clz(P > 1 ? P : 1);  // 0..15
        keys[q] = ((15 - cls) << kSeqBits) | i;
      }
    }
    bitonic_sort(keys, np, xbuf);
#pragma unroll
    for (int q = 0; q < kSortSlots; ++q) {
      const int i = q * kAttnThreads + tid;
      if (i < np) perm[i] = keys[q];
    }
    __syncthreads();
    // facts and item prefix in processing order (gathered through registers,
    // written back in place after the scan's barrier)
    int g_ot[kPerMax], g_pl[kPerMax];
    local = 0;
#pragma unroll
    for (int q = 0; q < kPerMax; ++q) {
      const int k = j0 + q;
      items_q[q] = 0;
      g_ot[q] = 0;
      g_pl[q] = 0;
      if (k < j1) {
        const int j = perm[k] & ((1 << kSeqBits) - 1);
        g_ot[q] = ot[j];
        g_pl[q] = pl[j];
        const int P = g_pl[q];
        const int T = int(unsigned(g_ot[q]) >> kTreeSizeShift);
        items_q[q] = p.hkv * cdiv(T * p.group, kRowsPerPass) * (P > 0 ? cdiv(P, chunk) : 1);
        local += items_q[q];
      }
    }
    run = block_exclusive_scan(local, scratch, total);
#pragma unroll
    for (int q = 0; q < kPerMax; ++q) {
      const int k = j0 + q;
      if (k < j1) {
        ot[k] = g_ot[q];
        pl[k] = g_pl[q];
        cum[k] = run;
        run += items_q[q];
      }
    }
  }
  if (tid == 0) {
    cum[n] = total;
    if (flag && (p.tree_offsets[0] != 0 || p.tree_offsets[p.batch] != p.total_nodes))
      set_error(p.hdr, kErrBadTree);
  }
  __syncthreads();
  return total;
}

struct Item {
  int b, g, rp, s, grp;
  int chunk;  // prefix tokens per item of this launch
  SeqInfo si;
};

// Decode item li into (sequence, KV head, row pass, chunk) and the sequence's
// facts from the LDS table, without any global-memory read.  Items are
// numbered sequence by sequence, then KV head, row pass and chunk (chunk
// fastest), so the chunks of a group have consecutive numbers.
__device__ __forceinline__ Item decode_item(const Params& p, int chunk, const int* cum,
                                            const int* ot, const int* pl, const int* perm,
                                            int li) {
  Item it;
  it.chunk = chunk;
  int lo = 0, hi = p.batch;  // largest b with cum[b] <= li
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (cum[mid] <= li) lo = mid; else hi = mid;
  }
  it.b = perm[lo] & ((1 << kSeqBits) - 1);
  const unsigned o = unsigned(ot[lo]);
  it.si.off = int(o & ((1u << kTreeSizeShift) - 1u));
  it.si.T = int(o >> kTreeSizeShift);
  it.si.P = pl[lo];
  it.si.S = it.si.P > 0 ? cdiv(it.si.P, chunk) : 1;
  it.si.RP = cdiv(it.si.T * p.group, kRowsPerPass);
  it.si.items = cum[lo + 1] - cum[lo];
  const int local = li - cum[lo];
  it.s = local % it.si.S;
  const int t = local / it.si.S;
  it.rp = t % it.si.RP;
  it.g = t / it.si.RP;
  it.grp = (it.b * p.hkv + it.g) * p.rp_max + it.rp;
  return it;
}

// Decode item li of a one-sequence launch without a table: the tree is the
// whole of q's rows (offset 0, N nodes, both known to the host), the chunk
// count is the bound s_max from max_prefix_len, and the prefix length is
// read with the item's other values (si.P = -1 until then); a chunk past the
// actual prefix turns out empty.
__device__ __forceinline__ Item decode_single(const Params& p, int li) {
  Item it;
  it.chunk = p.chunk;
  it.b = 0;
  it.si.off = 0;
  it.si.T = p.total_nodes;
  it.si.P = -1;
  it.si.S = p.s_max;
  it.si.RP = cdiv(it.si.T * p.group, kRowsPerPass);
  it.si.items = p.hkv * it.si.RP * it.si.S;
  it.s = li % it.si.S;
  const int t = li / it.si.S;
  it.rp = t % it.si.RP;
  it.g = t / it.si.RP;
  it.grp = it.g * p.rp_max + it.rp;
  return it;
}

// =========================================================== prefix piece
// LDS of one workgroup: a ring of NS KV slots (declared in attn_kernel), the
// tree rows and the sequence table (dynamic), and SmemMisc.
template <typename T, int D>
struct Geo {
  static constexpr int ROWB = D * int(sizeof(T));          // bytes per K/V row
  static constexpr int KCH = ROWB / 16;                    // 16-byte chunks per row
  static constexpr int SWZ = (KCH < 16 ? KCH : 16) - 1;    // XOR swizzle of chunk index
  static constexpr int BLKB = kBlock * ROWB;               // bytes of one K (or V) block
  static constexpr int KI = BLKB / (kAttnWaves * 1024);    // DMA instructions per wave per tensor
  static constexpr int QCH = D / 4 * int(sizeof(T)) / 16;  // 16-byte chunks of the Q fragment
  static constexpr int DT = D / 16;                        // 16-wide head-dim tiles of O^T
  // ring slots (a K block and a V block each): the host gives each launch as
  // many as fit beside the tree rows and the sequence table in the 160 KB of
  // LDS of the one workgroup per CU, at most NSMAX
  static constexpr int NSMAX = kMaxRingSlots;
  static constexpr int SLOTB = 2 * BLKB;
  static_assert(KI >= 1 && BLKB % (kAttnWaves * 1024) == 0, "DMA split");
  static_assert(NSMAX * 2 * KI < 64, "vmcnt range");
};

// words of SmemMisc::hid: landing places of the hidden loads of an item's
// first round trip
constexpr int kHidSense = 0;                  // the group's sense word (thread 0)
constexpr int kHidOff = 1;                    // tree_offsets[0], [1] (wave 0, lanes 0 and 1)
constexpr int kHidP = 4;                      // the prefix length, per wave
// blocks a tree region (cache positions P .. P+T-1, T <= 256) can touch
constexpr int kRegionBlocks = kMaxTreeSplit / kBlock + 1;
constexpr int kHidBlk = kHidP + kAttnWaves;   // the tree region's block ids, per wave
constexpr int kHidStarted = kHidBlk + kRegionBlocks * kAttnWaves;  // the group's started count (thread 0)
constexpr int kHidWords = kHidStarted + 1;

struct SmemMisc {
  uint64_t mask[kMaxTree];
  int hid[kHidWords];
  int scratch[kAttnThreads];
  int bcast[4];
  int more[2];             // pointer jumping: some node still had a link after round r (slot r & 1)
  float half_m[kMaxTree];  // running max / sum of the upper key half, per row
  float half_l[kMaxTree];
};

// XOR key of row t's 16-byte chunks in a swizzled row-major tile: logical
// chunk c sits at physical chunk c ^ swz_key(t).  For bf16 rows of 16 chunks
// the key is a bit permutation of t (bits 0-2 move up one, bit 0 becomes
// bit 2 ^ bit 3), so that
//  - the K reads (16 consecutive rows at one chunk, 16 bytes a lane) hit 16
//    distinct chunks, also any 8 aligned rows 8 distinct chunks mod 8, and
//  - the transposing V reads (per 32 lanes: 8 aligned rows, two adjacent
//    chunks, 8 bytes a lane) cover all 16 chunks once: no two lanes of a pass
//    share a bank.  The plain key t & 15 put two lanes on each bank there.
// Other tiles keep the plain key.
template <typename T, int D>
__device__ __forceinline__ int swz_key(int t) {
  using Gm = Geo<T, D>;
  if constexpr (sizeof(T) == 2 && Gm::KCH == 16)
    return (((t >> 2) ^ (t >> 3)) & 1) | ((t & 7) << 1);
  else
    return t & Gm::SWZ;
}

// byte offset of logical 16-byte chunk c of row t in a swizzled row-major tile
template <typename T, int D>
__device__ __forceinline__ int swz_off(int t, int c) {
  using Gm = Geo<T, D>;
  return t * Gm::ROWB + ((c ^ swz_key<T, D>(t)) << 4);
}

// Direct global -> LDS transfers (16 bytes per lane, landing at lds_base + 16 *
// lane; lds_base wave-uniform) are written as inline assembly on purpose.  The
// compiler, when it sees them as LDS writes, cannot tell which LDS object an
// in-flight transfer targets and makes every later LDS read wait for all
// outstanding transfers, including the prefetched KV blocks, which would
// serialise the ring.  Here every wait is explicit: a slot is read only after
// a vmcnt wait that covers its transfers and a barrier.  M0 carries the LDS
// address and is set in the same statement.  The address-space cast exists
// only for the device target, so the host pass sees empty bodies.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
#if defined(__HIP_DEVICE_COMPILE__)
  return uint32_t(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const void*)p));
#else
  return uint32_t(reinterpret_cast<uintptr_t>(p));
#endif
}
// lane's 16 bytes from its own global address g
__device__ __forceinline__ void lds_dma16(const void* g, void* lds_base) {
#if defined(__HIP_DEVICE_COMPILE__)
  const uint32_t m0 = uint32_t(__builtin_amdgcn_readfirstlane(lds_addr(lds_base)));
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(m0), "v"(g) : "memory");
#endif
}

// Transposing 64-bit LDS read of 16-bit elements (ds_read_b64_tr_b16): inside
// each group of 16 lanes, lane L receives element L of the 4 rows whose
// addresses lanes 4j..4j+3 supply (j = 0..3), i.e. a 4x16 -> 16x4 transpose.
__device__ __forceinline__ uint2 lds_read_tr16(const unsigned char* a) {
#if defined(__HIP_DEVICE_COMPILE__)
  typedef short v4i16 __attribute__((ext_vector_type(4)));
  const v4i16 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) v4i16*)(const_cast<unsigned char*>(a)));
  return __builtin_bit_cast(uint2, r);
#else
  (void)a;
  return uint2{0, 0};
#endif
}

// Source byte offsets, within one 64-token K or V tile, of the 16-byte chunks
// this lane moves: instruction i of wave w fills LDS chunks (w KI + i) 64 +
// lane, i.e. row t, physical chunk pc, which holds logical chunk pc ^ swz_key(t).
template <typename T, int D>
__device__ __forceinline__ void dma_offsets(uint32_t* off) {
  using Gm = Geo<T, D>;
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
#pragma unroll
  for (int i = 0; i < Gm::KI; ++i) {
    const int u = (w * Gm::KI + i) * 64 + lane;
    const int t = u / Gm::KCH;
    const int pc = u % Gm::KCH;
    off[i] = uint32_t(t * Gm::ROWB + ((pc ^ swz_key<T, D>(t)) << 4));
  }
}

// DMA one 64-token K or V tile (64 x D, row-major, swizzled) into LDS; every
// wave moves KI kilobytes of it, to LDS addresses m0, m0 + 1024, ... (m0
// wave-uniform, already offset for this wave).  `g` is wave-uniform.  The
// per-lane offsets stay in the same registers for the whole item, so no
// instruction writes a register that a transfer still in flight names (the
// compiler would make it wait for every outstanding transfer first).
template <typename T, int D>
__device__ __forceinline__ void dma_block(const unsigned char* g, uint32_t m0, const uint32_t* off) {
#if defined(__HIP_DEVICE_COMPILE__)
  using Gm = Geo<T, D>;
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  const uint64_t a = reinterpret_cast<uint64_t>(g);
  const u32x4 desc = {uint32_t(__builtin_amdgcn_readfirstlane(uint32_t(a))),
                      uint32_t(__builtin_amdgcn_readfirstlane(uint32_t(a >> 32) & 0xffffu)),
                      uint32_t(Gm::BLKB), 0x00020000u};
#pragma unroll
  for (int i = 0; i < Gm::KI; ++i)
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds" ::"s"(m0 + 1024u * i),
                 "v"(off[i]), "s"(desc)
                 : "memory");
#endif
}

// A 32-bit global load hidden from the compiler, landing in LDS (lane i's
// word at lds_base + 4 i, lds_base wave-uniform) like the block transfers.
// Its value is read from LDS after the caller's own wait, so no compiler wait
// for it lands in front of the loads issued after it; and no register is
// written behind the compiler's back (a register the compiler spilled while
// such a load was in flight would keep its old value).
// kCoherentLoad reads past this XCD's L2, as an agent-scope load does.
template <bool kCoherentLoad = false>
__device__ __forceinline__ void hidden_load(const int* ptr, int* lds_base) {
#if defined(__HIP_DEVICE_COMPILE__)
  const uint32_t m0 = uint32_t(__builtin_amdgcn_readfirstlane(lds_addr(lds_base)));
  if constexpr (kCoherentLoad)
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, off sc1" ::"s"(m0), "v"(ptr) : "memory");
  else
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, off" ::"s"(m0), "v"(ptr) : "memory");
#endif
}

template <int n>
__device__ __forceinline__ void wait_vm() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (0x7 << 4) | (0xf << 8));
}
// Wait until at most k KV blocks (2 * KI DMA instructions each, the youngest
// memory operations of the wave) are still in flight; 0 <= k <= NS.
template <int KI, int NS>
__device__ __forceinline__ void wait_blocks(int k) {
  if (NS >= 4 && k >= 4) wait_vm<(NS >= 4 ? 8 * KI : 0)>();
  else if (NS >= 3 && k >= 3) wait_vm<(NS >= 3 ? 6 * KI : 0)>();
  else if (k >= 2) wait_vm<4 * KI>();
  else if (k == 1) wait_vm<2 * KI>();
  else wait_vm<0>();
}
// Barrier that does not drain outstanding loads (the caller waits for what it needs).
__device__ __forceinline__ void raw_barrier() {
  __builtin_amdgcn_s_waitcnt((0xf) | (0x3 << 14) | (0x7 << 4) | (0x0 << 8));  // lgkmcnt(0)
  __asm__ __volatile__("s_barrier" ::: "memory");
}

// Device-coherent accesses to the chunk partials.  The L2 of an XCD is not
// kept coherent with the others, and the chunks of a group may run on
// different XCDs, so partials are written and read with the sc1 cache policy
// (the one the compiler gives agent-scope atomic loads and stores) through a
// raw buffer descriptor over [base, base + bytes).
constexpr int kCoherent = 16;  // buffer cache-policy operand selecting sc1
__device__ __forceinline__ void coherent_store16(float* base, uint32_t bytes, uint32_t off,
                                                 floatx4 v) {
#if defined(__HIP_DEVICE_COMPILE__)
  typedef int v4i __attribute__((ext_vector_type(4)));
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4i, v),
                                         __builtin_amdgcn_make_buffer_rsrc(base, 0, bytes, 0x00020000),
                                         int(off), 0, kCoherent);
#endif
}
__device__ __forceinline__ void coherent_store4(float* base, uint32_t bytes, uint32_t off, float v) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(int, v),
                                        __builtin_amdgcn_make_buffer_rsrc(base, 0, bytes, 0x00020000),
                                        int(off), 0, kCoherent);
#endif
}
__device__ __forceinline__ float4 coherent_load16(const float* base, uint32_t bytes, uint32_t off) {
#if defined(__HIP_DEVICE_COMPILE__)
  typedef int v4i __attribute__((ext_vector_type(4)));
  const v4i r = __builtin_amdgcn_raw_buffer_load_b128(
      __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(base), 0, bytes, 0x00020000), int(off), 0,
      kCoherent);
  return __builtin_bit_cast(float4, r);
#else
  return make_float4(0.f, 0.f, 0.f, 0.f);
#endif
}
__device__ __forceinline__ float coherent_load4(const float* base, uint32_t bytes, uint32_t off) {
#if defined(__HIP_DEVICE_COMPILE__)
  return __builtin_bit_cast(
      float, __builtin_amdgcn_raw_buffer_load_b32(
                 __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(base), 0, bytes, 0x00020000),
                 int(off), 0, kCoherent));
#else
  return 0.f;
#endif
}

// Slack (log2 units) by which a block's max may exceed the running reference
// max before the reference moves; weights stay <= 2^kRescaleSlack.
constexpr float kRescaleSlack = 8.f;

// One work item on the 8 waves of a workgroup.  Wave w takes row tile w % 4
// and key half w / 4 of every 64-key block, with its own online-softmax state;
// the two halves of a row tile are merged once, at the end of the item.
// SUFFIX: the tree piece of the split path on its own -- no prefix, the tree
// keys streamed through the ring in segments of 64 nodes, each under its
// word of the precomputed ancestor-or-self mask (p.mask_in), fp32 outputs.
template <typename T, int D, bool FUSED, bool SUFFIX = false, bool BIG = false, bool TWO = false>
__device__ __forceinline__ void process_item(const Params& p, unsigned char* ring,
                                             unsigned char* tree_lds,
                                             SmemMisc& sm, const Item& it, int slot_index,
                                             bool solo_combine) {
  using Gm = Geo<T, D>;
  constexpr int ROWB = Gm::ROWB, KCH = Gm::KCH, BLKB = Gm::BLKB, KI = Gm::KI,
                QCH = Gm::QCH, DT = Gm::DT, NSMAX = Gm::NSMAX;
  const int NS = p.ns;  // ring slots of this launch, 1..NSMAX
  constexpr bool kBf16 = sizeof(T) == 2;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform for the compiler too
  const int lr = lane & 15;
  const int kq = lane >> 4;

  SeqInfo si = it.si;
  const bool need_p = si.P < 0;  // one-sequence numbering: the prefix length is read below
  const int G = p.group;
  const int R = si.T * G;
  const int rlo = it.rp * kRowsPerPass;
  const int rcount = min(kRowsPerPass, R - rlo);
  const int RT = cdiv(rcount, 16);
  const size_t head_stride = size_t(kBlock) * D;  // elements per (block, head)
  // Wave roles: row tile rt and key part kp of every 64-key block.  With at
  // most two row tiles a block is cut into four 16-key parts (so that even a
  // single row tile keeps all four SIMDs busy), else into two 32-key halves.
  const int RTW = RT <= 1 ? 1 : (RT <= 2 ? 2 : 4);
  const int KP = RT <= 2 ? 4 : 2;
  const int rt = w % RTW;
  const int kp = w / RTW;
  const bool active = rt < RT && kp < KP;

  // ---- one round trip for every global value the item needs in registers:
  // the group's barrier phase, the Q fragment of this wave's row tile (lane
  // (row lr, group kq) holds the head-dim range [kq*D/4, (kq+1)*D/4) of its
  // row), the tree's parent array and, last, the chunk's block ids (lane j:
  // block j).  All of it is complete before the first LDS transfer is issued,
  // so no later wait for these values can hold up the transfers.
  // The group's meeting words, at places that do not depend on the call's
  // shape, so that calls of any shape can share a workspace.  Without tickets
  // every item number is below the grid size: the pair (arrival counter,
  // sense) of the group's first item number in the barrier region.  With
  // tickets: the group's arrival counter in the ticket-counter region, which
  // follows the barrier region (the sense word read below is then that of a
  // clamped index and goes unused).
  const int first_item = slot_index - it.s;
  unsigned* const bar = p.arrive + size_t(min(first_item, kBarrierSlots - 1)) * kCounterStride;
  unsigned* const sense = bar + kSenseWord;
  unsigned* const started = bar + kStartedWord;
  unsigned long long* const leaving = reinterpret_cast<unsigned long long*>(bar + kLeaveWord);
  unsigned* const counter =
      solo_combine ? p.arrive + size_t(kBarrierSlots) * kCounterStride + size_t(it.grp) : bar;
  // nothing of the previous item is still in flight (free for the first item):
  // a wait the compiler would otherwise place before reusing registers of the
  // previous item lands here, not between the loads of this trip
  wait_vm<0>();
  // hidden (sm.hid): a compiler wait for it would stall the loads below
  if constexpr (!SUFFIX && !TWO)
    if (tid == 0) hidden_load<true>(reinterpret_cast<const int*>(sense), &sm.hid[kHidSense]);
  uint4 qv[QCH];
  {
    const int r = 16 * rt + lr;
    if (active && r < rcount) {
      const int rr = rlo + r;
      const int h = it.g * G + rr % G;
      const uint4* src = reinterpret_cast<const uint4*>(
          static_cast<const T*>(p.q) + (size_t(si.off + rr / G) * p.hq + h) * D + kq * (D / 4));
#pragma unroll
      for (int c = 0; c < QCH; ++c) qv[c] = src[c];
    } else {
#pragma unroll
      for (int c = 0; c < QCH; ++c) qv[c] = make_uint4(0, 0, 0, 0);
    }
  }
  // the parent array (the tree chunk needs it; in a one-sequence launch which
  // chunk that is is known only with the prefix length, so every chunk reads it)
  int par = -1;
  // (more than 64 nodes: thread i reads node i's parent)
  if (FUSED && (BIG ? tid < kMaxTreeSplit : w == 0) && (need_p || it.s == si.S - 1))
    par = p.parents[si.off + min(BIG ? tid : lane, si.T - 1)];
  // tree rows kept in the cache right after the prefix (positions P .. P+T-1,
  // at most nreg_max = T_max / 64 + 1 blocks).  The region starts inside this
  // chunk's block range or right after it, so nreg_max more lanes of the
  // block-id load below cover its blocks (lanes cpb .. cpb + nreg_max - 1 of
  // the id vector), also before P is known.  When the chunk leaves too few
  // spare lanes, lanes 0 .. nreg_max - 1 of every wave read the region's ids
  // (such launches use the sequence table, so P is known here).
  const int cpb = it.chunk / kBlock;  // blocks per chunk
  const int nreg_max = cdiv(p.max_tree, kBlock) + 1;
  const bool extra_lanes = FUSED && p.tree_in_cache && cpb + nreg_max <= 64;
  const bool tree_blk_here = FUSED && p.tree_in_cache && !extra_lanes && it.s == si.S - 1;
  if (tree_blk_here && lane < nreg_max)
    hidden_load(p.block_table + size_t(it.b) * p.max_blocks + min(si.P / kBlock + lane, p.max_blocks - 1),
                &sm.hid[kHidBlk + kRegionBlocks * w]);
  // one-sequence numbering: the prefix length, and (first item only) the two
  // tree offsets, which must be 0 and N
  const bool first_of_launch = it.s == 0 && it.g == 0 && it.rp == 0;
  if (need_p) {
    if (lane == 0) hidden_load(p.prefix_lens, &sm.hid[kHidP + w]);
    if (first_of_launch && w == 0 && lane < 2) hidden_load(p.tree_offsets + lane, &sm.hid[kHidOff]);
  }
  int my_id = -1;
  if constexpr (!SUFFIX) {
    const int lb = it.s * cpb + lane;
    if (lane < cpb + (extra_lanes ? nreg_max : 0) && lb < p.max_blocks)
      my_id = p.block_table[size_t(it.b) * p.max_blocks + lb];
  }
  // suffix: this lane's row's mask words, one per 64-node segment
  constexpr int kSegMax = kMaxTreeSplit / 64;
  uint64_t segw[kSegMax] = {};
  if constexpr (SUFFIX) {
    const int r = 16 * rt + lr;
    if (active && r < rcount) {
      const size_t node = size_t(si.off + (rlo + r) / G);
#pragma unroll
      for (int sg = 0; sg < kSegMax; ++sg)
        if (sg < p.mask_words) segw[sg] = p.mask_in[node * p.mask_words + sg];
    }
  }
  wait_vm<0>();
  const unsigned sense0 = tid == 0 ? unsigned(sm.hid[kHidSense]) : 0u;  // used by thread 0 only
  const int tree_blk = tree_blk_here && lane < nreg_max ? sm.hid[kHidBlk + kRegionBlocks * w + lane] : 0;
  if (need_p) {
    const int p_read = __builtin_amdgcn_readfirstlane(sm.hid[kHidP + w]);  // the same in every lane
    const int toff = first_of_launch && w == 0 && lane < 2 ? sm.hid[kHidOff + lane] : 0;
    if (first_of_launch && w == 0 && lane < 2 && toff != (lane == 0 ? 0 : si.T))
      set_error(p.hdr, kErrBadTree);
    const bool p_ok = p_read >= 0 && p_read <= p.max_prefix;
    if (!p_ok && tid == 0 && first_of_launch) set_error(p.hdr, kErrBadPrefix);
    si.P = p_ok ? p_read : 0;
    si.S = si.P > 0 ? cdiv(si.P, it.chunk) : 1;
    if (it.s >= si.S) return;  // a chunk past the actual prefix
  }
  const int t0 = it.s * it.chunk;
  const int ntok = max(0, min(si.P, t0 + it.chunk) - t0);
  const int nblk = cdiv(ntok, kBlock);
  const int S = si.S;
  const bool with_tree = FUSED && it.s == S - 1;  // the last chunk also attends to the tree
  // The chunks of a first-round group of several chunks meet after their
  // partials are written.  Each counts itself as started here, once its
  // chunk is known to be non-empty and before its first KV transfer, so
  // that the meeting can tell whether every chunk of the group is running.
  const bool meet = !SUFFIX && !solo_combine && S > 1 && !TWO;
  if (meet && tid == 0) __hip_atomic_fetch_add(started, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  // trees of more than 64 nodes (fused): their 64-node segments follow the
  // chunk's KV blocks through the ring, under mask words built in LDS
  constexpr bool big = FUSED && BIG;

  // ---- tree rows (fused, last chunk only): DMA into LDS, issued before the KV
  // blocks so that waiting for them does not wait for the blocks.  Every
  // staged row past the tree holds a copy of its last node, so all staged rows
  // are finite.
  unsigned char* tk = tree_lds;
  unsigned char* tv = tree_lds + p.tree_lds_half;
  const int tree_rows = (SUFFIX || big) ? kBlock : p.tree_lds_half / ROWB;  // staged rows (>= tree size)
  // in-cache rows: the region's block ids, lane k holding block k of the
  // region (checked; bad ids are flagged and read as block 0)
  int regv = 0;
  if (with_tree && p.tree_in_cache) {
    const int nreg = (si.P + si.T - 1) / kBlock - si.P / kBlock + 1;
    if (extra_lanes) {
      const int r0 = si.P / kBlock - it.s * cpb;  // 0 .. cpb
      regv = __shfl(my_id, min(r0 + lane, 63));
    } else {
      regv = tree_blk;
    }
    const bool ok = (si.P + si.T - 1) / kBlock < p.max_blocks &&
                    __all(lane >= nreg || (regv >= 0 && regv < p.num_blocks));
    if (!ok) {
      if (tid == 0) set_error(p.hdr, kErrBadPrefix);
      regv = 0;
    }
  }
  // block of cache position pos of the region (wave-wide shuffle)
  auto region_block = [&](int pos) { return __shfl(regv, pos / kBlock - si.P / kBlock); };
  if (with_tree && !big) {
    const int Tn = si.T;
    const int ninstr = p.tree_lds_half / 1024;
    for (int m = w; m < ninstr; m += kAttnWaves) {
      const int u = m * 64 + lane;
      const int t = min(u / KCH, Tn - 1);
      const int pc = u % KCH;
      const int c = pc ^ swz_key<T, D>(u / KCH);
      size_t roff;
      const T* kb;
      const T* vb;
      if (p.tree_in_cache) {
        const int pos = si.P + t;
        const int blk = region_block(pos);
        roff = ((size_t(blk) * p.hkv + it.g) * kBlock + (pos % kBlock)) * D;
        kb = static_cast<const T*>(p.k_cache);
        vb = static_cast<const T*>(p.v_cache);
      } else {
        roff = (size_t(si.off + t) * p.hkv + it.g) * D;
        kb = static_cast<const T*>(p.k_tree);
        vb = static_cast<const T*>(p.v_tree);
      }
      const unsigned char* gk = reinterpret_cast<const unsigned char*>(kb + roff);
      const unsigned char* gv = reinterpret_cast<const unsigned char*>(vb + roff);
      lds_dma16(gk + c * 16, tk + m * 1024);
      lds_dma16(gv + c * 16, tv + m * 1024);
    }
  }

  // ---- KV blocks -> LDS ring: block j sits in slot j % NS.  A block id out
  // of range is flagged, its DMA reads block 0 instead and the block counts
  // as empty (bit j of `bad`).
  constexpr int SLOTB = Gm::SLOTB;  // K tile, then V tile
  uint32_t doff[KI];
  dma_offsets<T, D>(doff);
  const uint64_t bad = __ballot(lane < nblk && !(my_id >= 0 && my_id < p.num_blocks));
  if (bad != 0 && tid == 0) set_error(p.hdr, kErrBadPrefix);
  // Block j goes to ring slot sl (= j % NS, which the callers keep as a
  // counter).  Every address here is wave-uniform and in scalar registers: the
  // block id comes by readlane, and the LDS side is this wave's part of the
  // slot as a 32-bit LDS address.
  const uint32_t ring_m0 =
      uint32_t(__builtin_amdgcn_readfirstlane(lds_addr(ring))) +
      uint32_t(__builtin_amdgcn_readfirstlane(w)) * uint32_t(KI * 1024);
  const size_t blk_stride = size_t(p.hkv) * head_stride;  // elements per pool block
  const size_t head_off = size_t(it.g) * head_stride;
  auto issue = [&](int j, int sl) {
    int id = __builtin_amdgcn_readlane(my_id, j);  // wave-uniform
    if ((bad >> j) & 1) id = 0;
    const uint32_t m0 = ring_m0 + uint32_t(sl) * uint32_t(SLOTB);
    const size_t base = size_t(uint32_t(id)) * blk_stride + head_off;
    dma_block<T, D>(reinterpret_cast<const unsigned char*>(static_cast<const T*>(p.k_cache) + base), m0, doff);
    dma_block<T, D>(reinterpret_cast<const unsigned char*>(static_cast<const T*>(p.v_cache) + base), m0 + BLKB, doff);
  };
  // tree segments (64 nodes each) go through the ring like KV blocks, after
  // the item's KV blocks (ring unit nblk + segment): in the split path's
  // suffix mode, and in the fused kernel's last chunk for trees of more than
  // 64 nodes.  Each stages the segment's rows, clamped to the last node,
  // gathered from the [node, KV head, D] tree tensors, or from the cache
  // positions P + node when the tree rows sit in the cache: KI transfers per
  // wave and tensor, like a KV block.
  const int nseg = (SUFFIX || (with_tree && big)) ? cdiv(si.T, kBlock) : 0;
  const int ntot = nblk + nseg;  // ring units of the item
  auto stage = [&](int j, int sl) {
    const int sg = j - nblk;
    unsigned char* sk = ring + sl * SLOTB;
    for (int m = w; m < BLKB / 1024; m += kAttnWaves) {
      const int u = m * 64 + lane;
      const int t = min(kBlock * sg + u / KCH, si.T - 1);
      const int pc = u % KCH;
      const int c = pc ^ swz_key<T, D>(u / KCH);
      size_t roff;
      const T* kb;
      const T* vb;
      if (FUSED && p.tree_in_cache) {
        const int pos = si.P + t;
        roff = ((size_t(region_block(pos)) * p.hkv + it.g) * kBlock + (pos % kBlock)) * D;
        kb = static_cast<const T*>(p.k_cache);
        vb = static_cast<const T*>(p.v_cache);
      } else {
        roff = (size_t(si.off + t) * p.hkv + it.g) * D;
        kb = static_cast<const T*>(p.k_tree);
        vb = static_cast<const T*>(p.v_tree);
      }
      lds_dma16(reinterpret_cast<const unsigned char*>(kb + roff) + c * 16, sk + m * 1024);
      lds_dma16(reinterpret_cast<const unsigned char*>(vb + roff) + c * 16, sk + BLKB + m * 1024);
    }
  };
  auto issue_any = [&](int j, int sl) {
    if (j < nblk) issue(j, sl);
    else stage(j, sl);
  };
  for (int j = 0; j < NS && j < ntot; ++j) issue_any(j, j);

  // ---- tree staging: wait for the tree DMA (older than the blocks), then the
  // tree mask by pointer jumping (as in tree_mask_wave)
  if (with_tree && big) {
    // node i (thread i) keeps its ancestor-or-self set in kSegMax words and a
    // link to an ancestor; rounds through LDS OR in the linked node's set and
    // follow its link, until no node has a link left (at most eight rounds).
    // Words of node i end at bw[i * kSegMax ..].
    uint64_t* bw = reinterpret_cast<uint64_t*>(tree_lds);
    int* bup = reinterpret_cast<int*>(tree_lds + kMaxTreeSplit * kSegMax * sizeof(uint64_t));
    const int Tn = si.T;
    const bool node = tid < kMaxTreeSplit;
    const bool bad_i = node && tid < Tn && !(par == -1 || (par >= 0 && par < tid));
    int up = (node && tid < Tn && !bad_i) ? par : -1;
    uint64_t anc[kSegMax];
#pragma unroll
    for (int x = 0; x < kSegMax; ++x)
      anc[x] = (node && tid < Tn && tid / 64 == x) ? (uint64_t(1) << (tid % 64)) : 0;
    for (int round = 0; round < 8; ++round) {
      if (node) {
#pragma unroll
        for (int x = 0; x < kSegMax; ++x) bw[tid * kSegMax + x] = anc[x];
        bup[tid] = up;
      }
      if (tid == 0) sm.more[round & 1] = 0;
      __syncthreads();
      if (node && up >= 0) {
#pragma unroll
        for (int x = 0; x < kSegMax; ++x) anc[x] |= bw[up * kSegMax + x];
        up = bup[up];
        if (up >= 0) sm.more[round & 1] = 1;
      }
      __syncthreads();
      // no node has a link left: every set is complete (the other slot is
      // cleared only after the next round's first barrier, so all threads
      // read this one before it changes)
      if (sm.more[round & 1] == 0) break;
    }
    if (node) {
#pragma unroll
      for (int x = 0; x < kSegMax; ++x) bw[tid * kSegMax + x] = anc[x];
    }
    if (__syncthreads_or(bad_i) && tid == 0 && it.g == 0 && it.rp == 0) set_error(p.hdr, kErrBadTree);
  } else if (with_tree) {
    wait_blocks<KI, NSMAX>(min(nblk, NS));
    if (w == 0) {
      const int Tn = si.T;
      const bool bad_lane = lane < Tn && !(par == -1 || (par >= 0 && par < lane));
      int up = (lane < Tn && !bad_lane) ? par : -1;
      uint64_t anc = lane < Tn ? (uint64_t(1) << lane) : 0;
#pragma unroll
      for (int round = 0; round < 6; ++round) {
        const int src = up >= 0 ? up : lane;
        const uint32_t lo = __shfl(static_cast<uint32_t>(anc), src);
        const uint32_t hi = __shfl(static_cast<uint32_t>(anc >> 32), src);
        const int up2 = __shfl(up, src);
        if (up >= 0) {
          anc |= (static_cast<uint64_t>(hi) << 32) | lo;
          up = up2;
        }
      }
      sm.mask[lane] = anc;
      if (__any(bad_lane) && lane == 0 && it.g == 0 && it.rp == 0) set_error(p.hdr, kErrBadTree);
    }
  }

  float m_run = -INFINITY, l_run = 0.f;
  floatx4 oacc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) oacc[dt] = floatx4{0.f, 0.f, 0.f, 0.f};

  // zero the V rows past the prefix in a partial block (the cache may hold
  // anything there, and 0 * NaN would leak into the PV product)
  auto clear_tail = [&](unsigned char* slot, int nvalid) {
    unsigned char* vb = slot + BLKB;
    for (int u = tid; u < (kBlock - nvalid) * KCH; u += kAttnThreads) {
      const int t = nvalid + u / KCH;
      *reinterpret_cast<uint4*>(vb + swz_off<T, D>(t, u % KCH)) = make_uint4(0, 0, 0, 0);
    }
  };

  // This wave's KS keys (key part kp) of one 64-key block: a prefix block
  // (keys < nvalid visible) or, with kTree, the staged tree rows (key j
  // visible to a row iff bit j of its node's mask word is set; staged-row
  // reads are clamped to the staging area).  Lane (row lr, group kq) ends up
  // holding scores of keys kp KS + 16 a + 4 kq + i (a < KS / 16, i < 4).
  auto compute = [&](auto tree_tag, auto ks_tag, auto mask_tag, const unsigned char* kb,
                     const unsigned char* vb, int nvalid, uint64_t tword) {
    constexpr bool kTree = decltype(tree_tag)::value;
    constexpr bool kMasked = kTree || decltype(mask_tag)::value;  // else every key is visible
    constexpr int KS = decltype(ks_tag)::value;  // 16 or 32 keys
    constexpr int NA = KS / 16;                  // 16-key tiles
    const int kbase = kp * KS;
    auto krow = [&](int t) { return kTree ? min(t, tree_rows - 1) : t; };
    uint64_t word = 0;
    if constexpr (kTree) {
      const int r = 16 * rt + lr;
      word = (SUFFIX || big) ? tword : (r < rcount ? sm.mask[(rlo + r) / G] : 0);
    }
    // every LDS read of the block is issued before the first MFMA
    uint4 kf[NA][QCH];
#pragma unroll
    for (int a = 0; a < NA; ++a)
#pragma unroll
      for (int c = 0; c < QCH; ++c)
        kf[a][c] = *reinterpret_cast<const uint4*>(
            kb + swz_off<T, D>(krow(kbase + 16 * a + lr), kq * QCH + c));
    // V^T fragments (A operand of O^T += V^T P^T), read together with K so
    // that their latency overlaps the QK product and the softmax.
    // The transposing LDS read gives lane (d, group kq) four consecutive keys
    // of column d: one read makes the four k-slots of a 16-key MFMA, two make
    // the eight of a 32-key one.
    constexpr int NVF = kBf16 ? DT : 1;
    uint4 vf[NVF];
    if constexpr (kBf16) {
      const int L = lane & 15;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        uint2 half[NA];
#pragma unroll
        for (int h = 0; h < NA; ++h) {
          const int row = krow(kbase + 16 * h + 4 * kq + (L >> 2));
          const int cb = 32 * dt + 8 * (L & 3);  // byte column
          half[h] = lds_read_tr16(vb + row * ROWB + (((cb >> 4) ^ swz_key<T, D>(row)) << 4) + (cb & 15));
        }
        if constexpr (NA == 2) vf[dt] = make_uint4(half[0].x, half[0].y, half[1].x, half[1].y);
        else vf[dt] = make_uint4(half[0].x, half[0].y, 0u, 0u);
      }
    }
    // keep every read above this point: one LDS round trip per block
    __builtin_amdgcn_sched_barrier(0);
    floatx4 sacc[NA];
#pragma unroll
    for (int a = 0; a < NA; ++a) sacc[a] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < QCH; ++c)
#pragma unroll
      for (int a = 0; a < NA; ++a) {
        if constexpr (kBf16) {
          sacc[a] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              __builtin_bit_cast(bf16x8, kf[a][c]), __builtin_bit_cast(bf16x8, qv[c]), sacc[a],
              0, 0, 0);
        } else {
          const uint4 kv = kf[a][c];
          const float ka[4] = {__builtin_bit_cast(float, kv.x), __builtin_bit_cast(float, kv.y),
                               __builtin_bit_cast(float, kv.z), __builtin_bit_cast(float, kv.w)};
          const float qa[4] = {__builtin_bit_cast(float, qv[c].x), __builtin_bit_cast(float, qv[c].y),
                               __builtin_bit_cast(float, qv[c].z), __builtin_bit_cast(float, qv[c].w)};
#pragma unroll
          for (int e = 0; e < 4; ++e)
            sacc[a] = __builtin_amdgcn_mfma_f32_16x16x4f32(ka[e], qa[e], sacc[a], 0, 0, 0);
        }
      }
    // Online softmax in base 2.  Scores stay unscaled until the exponent; the
    // running reference max m_run is in scaled units.  Only a partial block or
    // the tree block needs the per-key mask.
    const float c = p.scale_log2;
    float sr[NA][4];
    float rmax = -INFINITY;
#pragma unroll
    for (int a = 0; a < NA; ++a)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float v = sacc[a][i];
        if constexpr (kMasked) {
          const int tok = kbase + 16 * a + 4 * kq + i;
          const bool vis = kTree ? bool((word >> tok) & 1) : tok < nvalid;
          v = vis ? v : -INFINITY;
        }
        sr[a][i] = v;
        rmax = fmaxf(rmax, v);
      }
    rmax = max_over_quads(rmax);
    const float m_cand = rmax * c;  // -inf stays -inf (c > 0)
    // Move the reference only when this block's max exceeds it by more than
    // kRescaleSlack: the weights then stay <= 2^kRescaleSlack, and the costly
    // rescale of the running output is rare after the first block.  The
    // result does not depend on the reference (o / l and lse = m + log2 l).
    if (__any(m_cand > m_run + kRescaleSlack)) {
      const float m_new = m_cand > m_run + kRescaleSlack ? m_cand : m_run;
      const float alpha = m_new == m_run ? 1.f : exp2_fast(m_run - m_new);  // 0 from -inf
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) oacc[dt] *= alpha;
      m_run = m_new;
    }
    const float m_use = m_run == -INFINITY ? 0.f : m_run;
    float pr[NA][4];
    float rsum = 0.f;
#pragma unroll
    for (int a = 0; a < NA; ++a)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        // the denominator takes the fp32 weight, so the row's lse is exact to
        // fp32 rounding; only the PV operand is rounded to bf16
        const float e = exp2_fast(fmaf(sr[a][i], c, -m_use));
        pr[a][i] = e;
        rsum += e;
      }
    rsum = sum_over_quads(rsum);
    l_run += rsum;

    if constexpr (kBf16) {
      if constexpr (NA == 2) {
        bf16x8 bp;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          bp[i] = static_cast<__bf16>(pr[0][i]);
          bp[4 + i] = static_cast<__bf16>(pr[1][i]);
        }
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
          oacc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, vf[dt]), bp,
                                                             oacc[dt], 0, 0, 0);
      } else {
        typedef short v4i16 __attribute__((ext_vector_type(4)));
        v4i16 bp;
#pragma unroll
        for (int i = 0; i < 4; ++i) bp[i] = short(f32_to_bf16(pr[0][i]));
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const uint2 va = make_uint2(vf[dt].x, vf[dt].y);
          oacc[dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(v4i16, va), bp,
                                                               oacc[dt], 0, 0, 0);
        }
      }
    } else {
      // fp32: A operand V^T[16dt + lr][key], one element per MFMA; k-slot kq of
      // MFMA (a, i) is key kbase + 16 a + 4 kq + i
#pragma unroll
      for (int a = 0; a < NA; ++a)
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int row = krow(kbase + 16 * a + 4 * kq + i);
            const int cb = (16 * dt + lr) * 4;
            const float av = *reinterpret_cast<const float*>(
                vb + row * ROWB + (((cb >> 4) ^ swz_key<T, D>(row)) << 4) + (cb & 15));
            oacc[dt] = __builtin_amdgcn_mfma_f32_16x16x4f32(av, pr[a][i], oacc[dt], 0, 0, 0);
          }
    }
  };
  // ---- stream blocks [j0, j1) of the chunk through the ring; the DMA of
  // block j + NS starts as soon as every wave is done with block j.  The part
  // size, the per-key mask and whether this wave computes at all are fixed
  // for the whole loop, so the running output stays in place in registers.
  auto stream = [&](auto ks_tag, auto mask_tag, auto act_tag, int j0, int j1) {
    constexpr bool kMasked = decltype(mask_tag)::value;
    int sl = j0 % NS;  // ring slot of block j
    for (int j = j0; j < j1; ++j) {
      unsigned char* slot = ring + sl * SLOTB;
      wait_blocks<KI, NSMAX>(min(NS - 1, ntot - 1 - j));
      raw_barrier();
      int nv = kBlock;
      if constexpr (kMasked) {
        nv = ((bad >> j) & 1) ? 0 : min(kBlock, ntok - j * kBlock);
        if (nv < kBlock) {
          clear_tail(slot, nv);
          raw_barrier();
        }
      }
      if constexpr (decltype(act_tag)::value)
        compute(std::false_type{}, ks_tag, mask_tag, slot, slot + BLKB, nv, 0);
      raw_barrier();
      if (j + NS < ntot) issue_any(j + NS, sl);  // into the slot just freed
      sl = sl + 1 == NS ? 0 : sl + 1;
    }
  };
  // the tree piece (while the first KV blocks are still in flight), then the
  // full blocks without the per-key mask and a partial last block with it;
  // a chunk with a bad block id takes the masked loop throughout
  // the tree's segments after the KV blocks (trees of more than 64 nodes),
  // each under its mask word from LDS
  auto big_segments = [&](auto ks_tag, auto act_tag) {
    const uint64_t* bw = reinterpret_cast<const uint64_t*>(tree_lds);
    int sl = nblk % NS;
    for (int j = nblk; j < ntot; ++j) {
      unsigned char* slot = ring + sl * SLOTB;
      wait_blocks<KI, NSMAX>(min(NS - 1, ntot - 1 - j));
      raw_barrier();
      const int r = 16 * rt + lr;
      const uint64_t word = r < rcount ? bw[((rlo + r) / G) * kSegMax + (j - nblk)] : 0;
      if constexpr (decltype(act_tag)::value)
        compute(std::true_type{}, ks_tag, std::true_type{}, slot, slot + BLKB, 0, word);
      raw_barrier();
      if (j + NS < ntot) issue_any(j + NS, sl);
      sl = sl + 1 == NS ? 0 : sl + 1;
    }
  };
  auto tree_and_stream = [&](auto ks_tag, auto act_tag) {
    if (with_tree && !big) {
      raw_barrier();  // staged rows of every wave and the mask words are in LDS
      // a key part past the tree's last node sees no key of the tree block
      // (on the 8k verify with one KV head and 5 query heads the tree chunk
      // is the launch's slowest: 12.65 to 12.54 us a call)
      if constexpr (decltype(act_tag)::value)
        if (kp * decltype(ks_tag)::value < si.T)
          compute(std::true_type{}, ks_tag, std::true_type{}, tk, tv, 0, 0);
    }
    if (bad != 0) {
      stream(ks_tag, std::true_type{}, act_tag, 0, nblk);
    } else {
      const int nfull = ntok / kBlock;
      stream(ks_tag, std::false_type{}, act_tag, 0, nfull);
      stream(ks_tag, std::true_type{}, act_tag, nfull, nblk);
    }
    if (with_tree && big) big_segments(ks_tag, act_tag);
  };
  auto segments = [&](auto ks_tag, auto act_tag) {
    // unrolled, so that segw is indexed by constants and stays in registers
    int sl = 0;
#pragma unroll
    for (int sg = 0; sg < kSegMax; ++sg) {
      if (sg >= nseg) break;
      unsigned char* slot = ring + sl * SLOTB;
      wait_blocks<KI, NSMAX>(min(NS - 1, nseg - 1 - sg));
      raw_barrier();
      if constexpr (decltype(act_tag)::value)
        compute(std::true_type{}, ks_tag, std::true_type{}, slot, slot + BLKB, 0, segw[sg]);
      raw_barrier();
      if (sg + NS < nseg) issue_any(sg + NS, sl);
      sl = sl + 1 == NS ? 0 : sl + 1;
    }
  };
  if constexpr (SUFFIX) {
    if (KP == 4) {
      if (active) segments(std::integral_constant<int, 16>{}, std::true_type{});
      else segments(std::integral_constant<int, 16>{}, std::false_type{});
    } else {
      if (active) segments(std::integral_constant<int, 32>{}, std::true_type{});
      else segments(std::integral_constant<int, 32>{}, std::false_type{});
    }
  } else if (KP == 4) {
    if (active) tree_and_stream(std::integral_constant<int, 16>{}, std::true_type{});
    else tree_and_stream(std::integral_constant<int, 16>{}, std::false_type{});
  } else {
    if (active) tree_and_stream(std::integral_constant<int, 32>{}, std::true_type{});
    else tree_and_stream(std::integral_constant<int, 32>{}, std::false_type{});
  }
  wait_vm<0>();
  __syncthreads();

  // ---- merge the key parts of each row tile, pairwise (part kp + half into
  // part kp), in one or two rounds; the lane-major exchange goes through ring
  // slot 0, which holds the 4 * DT * 64 float4 of one round in every geometry
  {
    floatx4* xo = reinterpret_cast<floatx4*>(ring);
    for (int half = KP / 2; half >= 1; half >>= 1) {
      if (active && kp >= half && kp < 2 * half) {
        const int e = (kp - half) * RTW + rt;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) xo[(e * DT + dt) * 64 + lane] = oacc[dt];
        if (kq == 0) {
          sm.half_m[16 * e + lr] = m_run;
          sm.half_l[16 * e + lr] = l_run;
        }
      }
      __syncthreads();
      if (active && kp < half) {
        const int e = kp * RTW + rt;
        const float m1 = sm.half_m[16 * e + lr];
        const float l1 = sm.half_l[16 * e + lr];
        const float M = fmaxf(m_run, m1);
        const float mu = M == -INFINITY ? 0.f : M;
        const float a0 = exp2_fast(m_run - mu);
        const float a1 = exp2_fast(m1 - mu);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) oacc[dt] = a0 * oacc[dt] + a1 * xo[(e * DT + dt) * 64 + lane];
        l_run = a0 * l_run + a1 * l1;
        m_run = M;
      }
      __syncthreads();
    }
  }

  // ---- a group with a single chunk: normalise and write its rows directly
  if (S == 1) {
    if (kp == 0 && active) {
      const int r = 16 * rt + lr;
      if (r < rcount) {
        const int rr = rlo + r;
        const size_t orow = size_t(si.off + rr / G) * p.hq + it.g * G + rr % G;
        const bool any = m_run != -INFINITY;
        const float inv = any ? 1.f / l_run : 0.f;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const floatx4 o = oacc[dt] * inv;
          const size_t e = orow * D + 16 * dt + 4 * kq;
          if constexpr (FUSED && kBf16) {
            const uint32_t lo = uint32_t(f32_to_bf16(o[0])) | (uint32_t(f32_to_bf16(o[1])) << 16);
            const uint32_t hi = uint32_t(f32_to_bf16(o[2])) | (uint32_t(f32_to_bf16(o[3])) << 16);
            *reinterpret_cast<uint2*>(static_cast<uint16_t*>(p.out) + e) = make_uint2(lo, hi);
          } else {
            *reinterpret_cast<floatx4*>(static_cast<float*>(p.out) + e) = o;
          }
        }
        if (kq == 0 && p.lse_out)
          p.lse_out[orow] = any ? (m_run + __log2f(l_run)) * kLn2 : -INFINITY;
      }
    }
    return;
  }

  // ---- chunk partial -> workspace (device-coherent stores): the fp32 o rows
  // (D floats each), then the running max m and sum l of every row.  The o
  // rows are first gathered in LDS (16-byte pieces XOR-swizzled by row
  // against bank conflicts), so that the stores to the workspace cover whole
  // cache lines: lane i stores bytes [16 i, 16 i + 16) of the slot's o rows.
  {
    constexpr int PER_ROW = D / 4;  // 16-byte pieces per o row
    static_assert(kRowsPerPass * D * 4 <= Gm::SLOTB, "staged o rows fit one ring slot");
    unsigned char* stage = ring;    // free once the key parts are merged
    float* slotp = p.partials + size_t(slot_index) * p.slot_floats;
    const uint32_t sbytes = uint32_t(p.slot_floats) * 4u;
    // the group's started count, read while the partial is being stored
    // (hidden, like the sense word: it lands in LDS and is read after the
    // wait below)
    if (meet && tid == 0) hidden_load<true>(reinterpret_cast<const int*>(started), &sm.hid[kHidStarted]);
    __syncthreads();
    if (kp == 0 && active) {
      const int r = 16 * rt + lr;
      if (r < rcount) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
          *reinterpret_cast<floatx4*>(stage + (r * PER_ROW + ((4 * dt + kq) ^ (r & 15))) * 16) = oacc[dt];
        if (kq == 0) {
          coherent_store4(slotp, sbytes, uint32_t(p.rows_slot * D + r) * 4u, m_run);
          coherent_store4(slotp, sbytes, uint32_t(p.rows_slot * D + p.rows_slot + r) * 4u, l_run);
        }
      }
    }
    __syncthreads();
    for (int i = tid; i < rcount * PER_ROW; i += kAttnThreads) {
      const int r = i / PER_ROW;
      const int c = i % PER_ROW;
      coherent_store16(slotp, sbytes, uint32_t(i) * 16u,
                       *reinterpret_cast<const floatx4*>(stage + (r * PER_ROW + (c ^ (r & 15))) * 16));
    }
  }

  // two launches: combine_kernel, next on the stream, folds the partials
  if constexpr (TWO) return;

  // ---- meet the other chunks of the group.  The arrival counter goes from 0
  // to S, and the chunk that brings it to S resets it to 0 (ready for the next
  // call).  Every chunk's partial stores are complete before its arrival, so
  // they are all visible to whoever sees the counter reach S.
  //   solo_combine (items are handed out over several rounds, so the chunks
  //   of a group may run far apart in time): nobody waits; the chunk that
  //   arrives last combines every row of the group.
  //   otherwise (all chunks normally run at once): the S chunks split the
  //   rows of the combine, chunk s taking rows s, s + S, ...  A chunk waits
  //   for the others only when the started count it read shows every chunk
  //   of the group running: a running chunk always arrives, so that wait
  //   ends even when the launch does not hold the whole GPU (another kernel,
  //   or another verify call on another stream, may hold some of the CUs).
  //   Otherwise it records itself in the group's leaving mask before it
  //   arrives, and leaves.  The last arrival resets the counters, flips the
  //   group's sense word, which the waiting chunks poll (a sense-reversing
  //   barrier), and combines its own rows and those of every chunk that
  //   left, exactly as that chunk would have.
  wait_all_mem();  // this wave's partial stores are complete
  __syncthreads();
  uint64_t rows_of = uint64_t(1) << (it.s & 63);  // chunks whose rows this workgroup combines
  bool combine_all = false;
  if (solo_combine) {
    if (tid == 0) {
      const bool last = atomicAdd(counter, 1u) == unsigned(S - 1);
      if (last) __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      sm.bcast[2] = last;
    }
    __syncthreads();
    if (!sm.bcast[2]) return;
    combine_all = true;
  } else {
    if (tid == 0) {
      const unsigned st = unsigned(sm.hid[kHidStarted]);
      const bool leave = st < unsigned(S) || (p.force_leave && (it.s & 1));
      if (leave) {
        // complete before the arrival that publishes it
        __hip_atomic_fetch_or(leaving, 1ull << it.s, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        wait_all_mem();
      }
      unsigned long long extra = 0;
      int outcome = 0;  // 0: combine, 1: leave, 2: timed out
      if (atomicAdd(counter, 1u) == unsigned(S - 1)) {
        // every chunk has arrived, and every leaver's bit was set before its arrival
        extra = __hip_atomic_load(leaving, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(started, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (extra) __hip_atomic_store(leaving, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(sense, sense0 ^ 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      } else if (leave) {
        outcome = 1;
      } else {
        unsigned spins = 0;
        while (ld_counter(sense) == sense0) {
          __builtin_amdgcn_s_sleep(1);
          if (++spins > kSpinLimit) {
            outcome = 2;
            break;
          }
        }
        if (outcome == 2) set_error(p.hdr, kErrTimeout);
      }
      sm.bcast[2] = outcome;
      sm.bcast[0] = int(uint32_t(extra));
      sm.bcast[1] = int(uint32_t(extra >> 32));
    }
    __syncthreads();
    if (sm.bcast[2]) return;
    rows_of |= (uint64_t(uint32_t(sm.bcast[1])) << 32) | uint32_t(sm.bcast[0]);
  }

  // ---- combine.  This workgroup takes rows r0, r0 + rstride, ... of the
  // group (rows s, s + S, ... when the S chunks split the combine; every row
  // when it combines alone).  For one row, D/4 lanes (a row slot) cover the head dim, 4
  // elements each; QG row slots split the S chunk partials between them (all
  // loads issued up front), then meet in LDS.  The chunk partials (in the fused
  // kernel the last chunk's also holds the tree piece) are folded with their
  // log-sum-exp weights.
  // [merge_attentions over disjoint KV chunks: pith.science verdict record,
  // pith_extraction.supporting_citations (Juravsky et al. 2024)]
  // QMAX: partial loads per lane.  The solo combine of a group with many
  // chunks takes four times as many, so that several rows go in each pass
  // (each pass is one device-coherent round trip).
  constexpr int kQBase = kMaxSplits / (kAttnThreads / (D / 4));
  auto combine = [&](auto qmax_tag, int r0, int rstride) {
    constexpr int L4 = D / 4;
    constexpr int NSLOT = kAttnThreads / L4;
    constexpr int QMAX = decltype(qmax_tag)::value;
    static_assert((NSLOT & (NSLOT - 1)) == 0, "row slots are a power of two");
    // QG row slots per row: enough that QMAX loads per lane cover the S
    // partials, and no more than lets all of this workgroup's rows go in one
    // pass
    int QG = 1;
    while (QG * QMAX < S) QG <<= 1;
    const int rows_here = cdiv(rcount - r0, rstride);
    while (2 * QG <= NSLOT && 2 * QG <= S && NSLOT / (2 * QG) >= rows_here) QG <<= 1;
    const int RB = NSLOT / QG;
    const int rs = tid / L4;  // row slot
    const int d4 = tid % L4;
    const int qg = rs % QG;
    const int rb = rs / QG;
    float* red_m = reinterpret_cast<float*>(ring);
    float* red_l = red_m + NSLOT;
    float* red_o = red_l + NSLOT;                            // [NSLOT][D]
    const float* g0 = p.partials + size_t(slot_index - it.s) * p.slot_floats;  // chunk 0's slot
    const uint32_t gbytes = uint32_t(S) * uint32_t(p.slot_floats) * 4u;
    const int moff = p.rows_slot * D;
    const int loff = moff + p.rows_slot;
    for (int k0 = 0; r0 + rstride * k0 < rcount; k0 += RB) {
      const int r = r0 + rstride * (k0 + rb);
      const bool valid = r < rcount;
      const int rr = rlo + r;
      float mq[QMAX], lq[QMAX];
      float4 oq[QMAX];
#pragma unroll
      for (int j = 0; j < QMAX; ++j) {
        const int q = qg + QG * j;
        if (valid && q < S) {
          const uint32_t so = uint32_t(q * p.slot_floats);
          mq[j] = coherent_load4(g0, gbytes, (so + moff + r) * 4u);
          lq[j] = coherent_load4(g0, gbytes, (so + loff + r) * 4u);
          oq[j] = coherent_load16(g0, gbytes, (so + r * D + 4 * d4) * 4u);
        } else {
          mq[j] = -INFINITY;
          lq[j] = 0.f;
          oq[j] = make_float4(0.f, 0.f, 0.f, 0.f);
        }
      }
      float mloc = -INFINITY;
#pragma unroll
      for (int j = 0; j < QMAX; ++j) mloc = fmaxf(mloc, mq[j]);
      if (d4 == 0) red_m[rs] = mloc;
      __syncthreads();
      // LDS reads in groups of four, each group issued before any of it is
      // used (index clamped into the row slots, result masked): QG / 4
      // round trips rather than QG
      float M = -INFINITY;
      for (int x0 = 0; x0 < QG; x0 += 4) {
        float v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) v[u] = red_m[(rb * QG + x0 + u) & (NSLOT - 1)];
#pragma unroll
        for (int u = 0; u < 4; ++u) M = x0 + u < QG ? fmaxf(M, v[u]) : M;
      }
      float L = 0.f;
      float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
      if (M != -INFINITY) {
#pragma unroll
        for (int j = 0; j < QMAX; ++j) {
          const float wq = exp2_fast(mq[j] - M);
          L = fmaf(wq, lq[j], L);
          acc.x = fmaf(wq, oq[j].x, acc.x);
          acc.y = fmaf(wq, oq[j].y, acc.y);
          acc.z = fmaf(wq, oq[j].z, acc.z);
          acc.w = fmaf(wq, oq[j].w, acc.w);
        }
      }
      *reinterpret_cast<float4*>(red_o + rs * D + 4 * d4) = acc;
      if (d4 == 0) red_l[rs] = L;
      __syncthreads();
      if (qg == 0 && valid) {
        float Lt = 0.f;
        float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
        for (int x0 = 0; x0 < QG; x0 += 4) {
          float lx[4];
          float4 ox[4];
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const int sx = (rb * QG + x0 + u) & (NSLOT - 1);
            lx[u] = red_l[sx];
            ox[u] = *reinterpret_cast<const float4*>(red_o + sx * D + 4 * d4);
          }
#pragma unroll
          for (int u = 0; u < 4; ++u)
            if (x0 + u < QG) {
              Lt += lx[u];
              o.x += ox[u].x; o.y += ox[u].y; o.z += ox[u].z; o.w += ox[u].w;
            }
        }
        float lse = -INFINITY;
        if (M != -INFINITY) {
          const float inv = 1.f / Lt;
          o.x *= inv; o.y *= inv; o.z *= inv; o.w *= inv;
          lse = (M + __log2f(Lt)) * kLn2;
        } else {
          o = make_float4(0.f, 0.f, 0.f, 0.f);
        }
        const size_t orow = size_t(si.off + rr / G) * p.hq + it.g * G + rr % G;
        if constexpr (FUSED) {
          T* dst = static_cast<T*>(p.out) + orow * D + 4 * d4;
          if constexpr (kBf16) {
            const uint32_t lo = uint32_t(f32_to_bf16(o.x)) | (uint32_t(f32_to_bf16(o.y)) << 16);
            const uint32_t hi = uint32_t(f32_to_bf16(o.z)) | (uint32_t(f32_to_bf16(o.w)) << 16);
            *reinterpret_cast<uint2*>(dst) = make_uint2(lo, hi);
          } else {
            *reinterpret_cast<float4*>(dst) = o;
          }
        } else {
          *reinterpret_cast<float4*>(static_cast<float*>(p.out) + orow * D + 4 * d4) = o;
        }
        if (d4 == 0 && p.lse_out) p.lse_out[orow] = lse;
      }
      __syncthreads();
    }
  };
  if (combine_all) {
    if (S > kQBase) combine(std::integral_constant<int, 4 * kQBase>{}, 0, 1);
    else combine(std::integral_constant<int, kQBase>{}, 0, 1);
  } else {
    // rows of chunk c: c, c + S, ... (this chunk's own, then any that left)
    while (rows_of) {
      const int c = __builtin_ctzll(rows_of);
      rows_of &= rows_of - 1;
      combine(std::integral_constant<int, kQBase>{}, c, S);
    }
  }
}

// TWO: a one-sequence launch in two launches (see combine_kernel); the
// chunks end at their partial stores.
template <typename T, int D, bool FUSED, bool BIG = false, bool TWO = false>
__global__ void __launch_bounds__(kAttnThreads, 1) attn_kernel(Params p) {
  using Gm = Geo<T, D>;
  // dynamic LDS: the KV ring (ns slots), the tree rows (K then V), the table
  extern __shared__ __attribute__((aligned(16))) int dyn[];
  __shared__ SmemMisc sm;
  unsigned char* ring = reinterpret_cast<unsigned char*>(dyn);
  unsigned char* tree_lds = ring + size_t(p.ns) * Gm::SLOTB;
  int* cum = reinterpret_cast<int*>(tree_lds + 2 * p.tree_lds_half);  // [batch + 1]
  int* ot = cum + p.batch + 1;           // [batch]
  int* pl = ot + p.batch;                // [batch]
  int* perm = pl + p.batch;              // [pow2 >= batch]
  const int tid = threadIdx.x;

  int items;
  int chunk = p.chunk;
  if (p.single) {
    items = p.single_items;  // the tree offsets are checked by the launch's first item
  } else {
    // the sort's exchange buffers use the ring, which holds no block yet
    static_assert(2 * kMaxBatch * sizeof(int) <= size_t(Gm::SLOTB), "sort buffers fit one ring slot");
    items = build_table(p, cum, ot, pl, perm, sm.scratch, reinterpret_cast<int*>(ring), chunk);
    // the same in every thread: say so, so that the item loop and the
    // decode's divisions stay scalar (config 3: 26.53 to 26.41 us)
    items = __builtin_amdgcn_readfirstlane(items);
    chunk = __builtin_amdgcn_readfirstlane(chunk);
  }

  // items in increasing order: first blockIdx.x, then from the ticket counter.
  // A workgroup waits only for the other chunks of its own group, whose
  // numbers are adjacent to its own, and a group has no more chunks than the
  // grid has workgroups, so every awaited chunk is taken and finished.
  int li = int(blockIdx.x);
  if (p.xcd_major && li < items) li = (li % 8) * (items / 8) + li / 8;
  const bool tickets = items > p.first_round;  // else the first round covers every item
  while (li < items) {
    const Item it = p.single ? decode_single(p, li) : decode_item(p, chunk, cum, ot, pl, perm, li);
    process_item<T, D, FUSED, false, BIG, TWO>(p, ring, tree_lds, sm, it, li, tickets);
    if (!tickets) break;
    __syncthreads();
    if (tid == 0) sm.bcast[0] = p.first_round + int(atomicAdd(&p.hdr->ticket, 1u));
    __syncthreads();
    li = sm.bcast[0];
  }
  if (!tickets) return;

  // the last workgroup to leave resets the ticket counter for the next call
  // (the group barriers reset themselves)
  __syncthreads();
  if (tid == 0) {
    const unsigned n = atomicAdd(&p.hdr->done, 1u);
    if (n == gridDim.x - 1) {
      __hip_atomic_store(&p.hdr->ticket, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(&p.hdr->done, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// ========================================================= combine kernel
// The split reduce of a one-sequence launch made in two launches: attn_kernel
// has stored every chunk's partial (unnormalised o rows, running max m and
// running sum l, base 2) in the chunk's slot, and this kernel folds them.
// [merge_attentions over disjoint KV chunks: pith.science verdict record,
// pith_extraction.supporting_citations (Juravsky et al. 2024)]
// For a row with partials (o_c, m_c, l_c), c < S:
//   M = max_c m_c,  w_c = 2^(m_c - M),  o = sum_c w_c o_c / sum_c w_c l_c,
//   lse = (M + log2 sum_c w_c l_c) ln 2  (o = 0, lse = -inf when M = -inf).
// Items are numbered as in attn_kernel's one-sequence launches: group
// t = g * RP + rp (KV head g, row pass rp) owns the slots t * S .. t * S + S - 1,
// of which the first cdiv(P, chunk) ran (P the actual prefix length).
// Workgroup w takes rows_per_wg = NSLOT / QG rows of group w / wpg: D / 4
// lanes (a row slot) cover one row's head dim, 4 elements each, and QG row
// slots split its S partials between them, QMAX loads per lane, all issued
// up front; the QG slots then meet in LDS.  OutT: the output element type
// (the shape's dtype for the fused verify, fp32 for the prefix pass).
// Plain scalar arguments rather than Params: the library is built with
// kernarg preloading, so they reach the SGPRs with the dispatch and the
// partial loads leave without waiting on a kernarg load.
template <typename OutT, int D>
__global__ void __launch_bounds__(kAttnThreads)
combine_kernel(const float* __restrict__ partials, const int* __restrict__ prefix_lens,
               OutT* __restrict__ out, float* __restrict__ lse_out, int S, int G,
               int total_nodes, int rows_slot, int hq, int max_prefix, int chunk) {
  constexpr int L4 = D / 4;
  constexpr int NSLOT = kAttnThreads / L4;
  constexpr int QMAX = kMaxSplits / NSLOT;  // QG * QMAX >= S for S <= kMaxSplits
  __shared__ float red_m[NSLOT];
  __shared__ float red_l[NSLOT];
  __shared__ __attribute__((aligned(16))) float red_o[NSLOT * D];
  const int tid = threadIdx.x;
  const int QG = combine_qg<D>(S);
  const int R = total_nodes * G;
  const int wpg = combine_wpg<D>(R, QG);
  const int slot_floats = slot_floats_of(rows_slot, D);
  const int RP = cdiv(R, kRowsPerPass);
  const int t = int(blockIdx.x) / wpg;
  const int rp = t % RP;
  const int g = t / RP;
  const int rlo = rp * kRowsPerPass;
  const int rcount = min(kRowsPerPass, R - rlo);
  const int rs = tid / L4;  // row slot
  const int d4 = tid % L4;
  const int qg = rs % QG;
  const int rb = rs / QG;
  const int r = (int(blockIdx.x) % wpg) * (NSLOT / QG) + rb;
  const bool valid = r < rcount;
  const float* g0 = partials + size_t(t) * size_t(S) * slot_floats;  // chunk 0's slot
  const uint32_t gbytes = uint32_t(S) * uint32_t(slot_floats) * 4u;
  const int moff = rows_slot * D;
  const int loff = moff + rows_slot;
  // The grid was sized from max_prefix_len; the actual prefix length, read in
  // the same trip as the partials, says which chunks ran: chunks past it
  // stored nothing this call (their slots hold older data), and with a single
  // chunk the attention kernel wrote the output rows itself.
  const int p_read = prefix_lens[0];
  float mq[QMAX], lq[QMAX];
  float4 oq[QMAX];
#pragma unroll
  for (int j = 0; j < QMAX; ++j) {
    const int q = qg + QG * j;
    if (valid && q < S) {
      const uint32_t so = uint32_t(q * slot_floats);
      mq[j] = coherent_load4(g0, gbytes, (so + moff + r) * 4u);
      lq[j] = coherent_load4(g0, gbytes, (so + loff + r) * 4u);
      oq[j] = coherent_load16(g0, gbytes, (so + r * D + 4 * d4) * 4u);
    } else {
      mq[j] = -INFINITY;
      lq[j] = 0.f;
      oq[j] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
  }
  const int P = p_read >= 0 && p_read <= max_prefix ? p_read : 0;  // as attn_kernel reads it
  const int s_run = P > 0 ? cdiv(P, chunk) : 1;
#pragma unroll
  for (int j = 0; j < QMAX; ++j)
    if (qg + QG * j >= s_run) {
      mq[j] = -INFINITY;
      lq[j] = 0.f;
      oq[j] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
  float mloc = -INFINITY;
#pragma unroll
  for (int j = 0; j < QMAX; ++j) mloc = fmaxf(mloc, mq[j]);
  if (s_run == 1) return;  // the same in every thread
  if (d4 == 0) red_m[rs] = mloc;
  __syncthreads();
  float M = -INFINITY;
  for (int x = 0; x < QG; ++x) M = fmaxf(M, red_m[rb * QG + x]);
  float L = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  if (M != -INFINITY) {
#pragma unroll
    for (int j = 0; j < QMAX; ++j) {
      const float wq = exp2_fast(mq[j] - M);
      L = fmaf(wq, lq[j], L);
      acc.x = fmaf(wq, oq[j].x, acc.x);
      acc.y = fmaf(wq, oq[j].y, acc.y);
      acc.z = fmaf(wq, oq[j].z, acc.z);
      acc.w = fmaf(wq, oq[j].w, acc.w);
    }
  }
  *reinterpret_cast<float4*>(red_o + rs * D + 4 * d4) = acc;
  if (d4 == 0) red_l[rs] = L;
  __syncthreads();
  if (qg != 0 || !valid) return;
  float Lt = 0.f;
  float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int x = 0; x < QG; ++x) {
    const int sx = rb * QG + x;
    Lt += red_l[sx];
    const float4 ox = *reinterpret_cast<const float4*>(red_o + sx * D + 4 * d4);
    o.x += ox.x;
    o.y += ox.y;
    o.z += ox.z;
    o.w += ox.w;
  }
  float lse = -INFINITY;
  if (M != -INFINITY) {
    const float inv = 1.f / Lt;
    o.x *= inv;
    o.y *= inv;
    o.z *= inv;
    o.w *= inv;
    lse = (M + __log2f(Lt)) * kLn2;
  } else {
    o = make_float4(0.f, 0.f, 0.f, 0.f);
  }
  const int rr = rlo + r;
  const size_t orow = size_t(rr / G) * hq + g * G + rr % G;
  OutT* dst = out + orow * D + 4 * d4;
  if constexpr (sizeof(OutT) == 2) {
    const uint32_t lo = uint32_t(f32_to_bf16(o.x)) | (uint32_t(f32_to_bf16(o.y)) << 16);
    const uint32_t hi = uint32_t(f32_to_bf16(o.z)) | (uint32_t(f32_to_bf16(o.w)) << 16);
    *reinterpret_cast<uint2*>(dst) = make_uint2(lo, hi);
  } else {
    *reinterpret_cast<float4*>(dst) = o;
  }
  if (d4 == 0 && lse_out) lse_out[orow] = lse;
}

// ============================================================ mask kernel
// One wave per sequence: mask_out[off + i] = ancestor-or-self word of node i.
__global__ void __launch_bounds__(64) mask_kernel(Params p, uint64_t* mask_out) {
  const int b = blockIdx.x;
  const int lane = threadIdx.x;
  const int o0 = p.tree_offsets[b];
  const int o1 = p.tree_offsets[b + 1];
  const int T = o1 - o0;
  const bool ok = o0 >= 0 && o1 >= o0 && o1 <= p.total_nodes && T <= p.max_tree;
  if (!ok) {
    if (lane == 0) set_error(p.hdr, kErrBadTree);
    return;
  }
  if (b == 0 && lane == 0 && (p.tree_offsets[0] != 0 || p.tree_offsets[p.batch] != p.total_nodes))
    set_error(p.hdr, kErrBadTree);
  bool bad = false;
  const uint64_t word = tree_mask_wave(p.parents + o0, T, bad);
  if (bad && lane == 0) set_error(p.hdr, kErrBadTree);
  if (lane < T) mask_out[o0 + lane] = bad ? 0 : word;
}

// One workgroup of 256 threads per sequence for trees of up to 256 nodes:
// thread i keeps node i's ancestor-or-self set in W <= 4 words and a link
// to an ancestor; each round ORs in the set of the linked node and follows
// its link (through LDS), doubling the distance covered, until no node has a
// link left (at most eight rounds).  Output
// mask_out[(off + i) * W + w], bit j % 64 of word j / 64.
__global__ void __launch_bounds__(kMaxTreeSplit) mask_words_kernel(Params p, uint64_t* mask_out) {
  __shared__ uint64_t anc_sh[kMaxTreeSplit * 4];
  __shared__ int up_sh[kMaxTreeSplit];
  __shared__ int more_sh[2];  // some node still had a link after round r (slot r & 1)
  __shared__ int bad_sh;
  const int b = blockIdx.x;
  const int i = threadIdx.x;
  const int W = p.mask_words;
  const int o0 = p.tree_offsets[b];
  const int o1 = p.tree_offsets[b + 1];
  const int T = o1 - o0;
  const bool ok = o0 >= 0 && o1 >= o0 && o1 <= p.total_nodes && T <= p.max_tree;
  if (!ok) {
    if (i == 0) set_error(p.hdr, kErrBadTree);
    return;
  }
  if (b == 0 && i == 0 && (p.tree_offsets[0] != 0 || p.tree_offsets[p.batch] != p.total_nodes))
    set_error(p.hdr, kErrBadTree);
  if (i == 0) bad_sh = 0;
  __syncthreads();
  int up = -1;
  uint64_t anc[4] = {0, 0, 0, 0};
  if (i < T) {
    const int pr = p.parents[o0 + i];
    const bool bad = !(pr == -1 || (pr >= 0 && pr < i));
    if (bad) bad_sh = 1;
    up = bad ? -1 : pr;
    anc[i / 64] = uint64_t(1) << (i % 64);
  }
  for (int round = 0; round < 8; ++round) {
#pragma unroll
    for (int w = 0; w < 4; ++w) anc_sh[i * 4 + w] = anc[w];
    up_sh[i] = up;
    if (i == 0) more_sh[round & 1] = 0;
    __syncthreads();
    if (up >= 0) {
#pragma unroll
      for (int w = 0; w < 4; ++w) anc[w] |= anc_sh[up * 4 + w];
      up = up_sh[up];
      if (up >= 0) more_sh[round & 1] = 1;
    }
    __syncthreads();
    if (more_sh[round & 1] == 0) break;  // no node has a link left
  }
  const bool bad = bad_sh != 0;
  if (bad && i == 0) set_error(p.hdr, kErrBadTree);
  if (i < T)
    for (int w = 0; w < W; ++w) mask_out[size_t(o0 + i) * W + w] = bad ? 0 : anc[w];
}

// ========================================================== suffix kernel
// The tree piece of the split path: one workgroup per (sequence, KV head,
// row pass), the item's rows against every tree node in 64-node segments
// under the precomputed mask words, on the MFMA path of the prefix kernel.
// Writes normalised o and natural-log lse (fp32).  Invalid tree offsets
// leave the sequence's rows unwritten.
// [draft-token piece that needs the tree mask: pith.science review,
// "What carries the argument"]
template <typename T, int D>
__global__ void __launch_bounds__(kAttnThreads, 1) suffix_kernel(Params p) {
  extern __shared__ __attribute__((aligned(16))) int dyn[];
  __shared__ SmemMisc sm;
  unsigned char* ring = reinterpret_cast<unsigned char*>(dyn);
  const int grp = blockIdx.x;
  Item it;
  it.rp = grp % p.rp_max;
  const int bg = grp / p.rp_max;
  it.g = bg % p.hkv;
  it.b = bg / p.hkv;
  it.s = 0;
  it.grp = grp;
  it.chunk = kBlock;
  const int o0 = p.tree_offsets[it.b];
  const int o1 = p.tree_offsets[it.b + 1];
  const int Tn = o1 - o0;
  if (!(o0 >= 0 && o1 > o0 && o1 <= p.total_nodes && Tn <= p.max_tree)) return;
  it.si.off = o0;
  it.si.T = Tn;
  it.si.P = 0;
  it.si.S = 1;
  it.si.RP = cdiv(Tn * p.group, kRowsPerPass);
  it.si.items = p.hkv * it.si.RP;
  if (it.rp >= it.si.RP) return;
  process_item<T, D, false, true>(p, ring, ring, sm, it, grp, false);
}

// =========================================================== merge kernel
template <typename OutT>
__global__ void __launch_bounds__(256) merge_kernel(long long rows, int D, const float* o_a,
                                                    const float* lse_a, const float* o_b,
                                                    const float* lse_b, OutT* out, float* lse_out) {
  const int per_row = D / 4;
  const long long n = rows * per_row;
  for (long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x; idx < n;
       idx += (long long)gridDim.x * blockDim.x) {
    const long long r = idx / per_row;
    const int c = int(idx % per_row) * 4;
    const float la = lse_a[r], lb = lse_b[r];
    const float m = fmaxf(la, lb);
    float4 res = make_float4(0.f, 0.f, 0.f, 0.f);
    float lse = -INFINITY;
    if (m != -INFINITY) {
      const float wa = expf(la - m), wb = expf(lb - m);
      const float tot = wa + wb;
      const float ca = wa / tot, cb = wb / tot;
      const float4 a = *reinterpret_cast<const float4*>(o_a + r * D + c);
      const float4 bb = *reinterpret_cast<const float4*>(o_b + r * D + c);
      res = make_float4(ca * a.x + cb * bb.x, ca * a.y + cb * bb.y, ca * a.z + cb * bb.z,
                        ca * a.w + cb * bb.w);
      lse = m + logf(tot);
    }
    OutT* dst = out + r * D + c;
    dst[0] = Elem<OutT>::from_f(res.x);
    dst[1] = Elem<OutT>::from_f(res.y);
    dst[2] = Elem<OutT>::from_f(res.z);
    dst[3] = Elem<OutT>::from_f(res.w);
    if (c == 0 && lse_out) lse_out[r] = lse;
  }
}

}  // namespace ta
