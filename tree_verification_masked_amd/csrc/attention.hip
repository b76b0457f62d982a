// Tree-masked split-KV GQA attention.
//
// Tree-verification notes (zhangshuibai.github.io), "Tree Verification 详解" part B:
// every flattened tree node attends to the prompt, its ancestors and itself, so its
// output equals an ordinary causal run of prompt + Path(root, node); part D.2: the
// node-to-prompt product is O(N * P) and dominates, the node-to-tree part is sparse.
// "EAGLE-4 Technical Deepdive" (blog.fal.ai), "EAGLE-4 verification trees and
// harness": the mask shows the shared prefix, the ancestors and the token itself.
//
// Work split: the logical key range [0, max_kv_len) is cut into S splits of whole
// 64-key tiles; a workgroup owns (request, KV head, query block, split) and keeps an
// online softmax per query row.  The rows of one KV head are its n_max * hq/hkv
// (node, query head) pairs, so K/V tiles are loaded once per workgroup and reused by
// every row (GQA).  Partials (max, sum, output divided by the sum, stored in the
// element type of the inputs) go to the workspace and
// a combine kernel merges the splits with a log-sum-exp rescale.
//
//  * MFMA path (bf16, >= 16 rows per KV head): eight waves, four row blocks of 32
//    rows, each block done by two waves that take the two 32-key halves of every
//    tile (their partial softmax states merge in LDS at the end).  Scores are
//    computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16, so each lane
//    ends up owning one query row; that accumulator layout is exactly the B operand
//    of O^T = V^T P^T for a fixed permutation of the 16 keys of a step, and V is
//    read transposed out of LDS in that key order.
//  * Shuffle path (fp32, or fewer than 16 rows): lane j of a wave scores key j of
//    the tile against one row, the row softmax uses wave reductions, and P V is
//    accumulated with one lane per head dimension.
#include <algorithm>
#include <mutex>
#include <type_traits>

#include "attn_combine.hpp"
#include "internal.hpp"

namespace spectree {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kTile = 64;           // keys per tile
constexpr int kMfmaRowsPerWg = 128; // 4 row blocks of 32 (each done by two waves, one per key half)
constexpr int kShflRowsPerWg = 16;  // 4 waves x 4 rows
constexpr int kMaxSplitPages = 1024;  // page ids of one split kept in LDS
constexpr float kLog2e = 1.4426950408889634f;


// A workgroup-uniform read of memory the launch never writes, through the constant
// address space: a scalar load, which no wait for the vector loads in flight covers.
template <typename T>
__device__ inline T uniform_read(const T* p) {
  return *(const __attribute__((address_space(4))) T*)p;
}

// Element offset of key t (< len) of request b, KV head g; -1 for a bad page id.
__device__ inline int64_t kv_off(const AttnArgs& a, int b, int t, int g) {
  if (!a.block_table) return (((int64_t)b * a.kv_capacity + t) * a.hkv + g) * a.head_dim;
  const int page = a.block_table[(int64_t)b * a.kv_capacity + t / a.page_size];
  if (page < 0 || page >= a.n_pages) return -1;
  return (((int64_t)page * a.page_size + t % a.page_size) * a.hkv + g) * a.head_dim;
}

__device__ inline bool key_visible(int t, int len, int ctx, uint64_t anc_row) {
  if (t >= len) return false;
  if (t < ctx) return true;
  return (anc_row >> (t - ctx)) & 1ull;
}

// ---------------------------------------------------------------------------
// MFMA path
// ---------------------------------------------------------------------------
// K and V tiles (64 keys) go from HBM straight into LDS with 16-byte
// global_load_lds, kStages tiles in flight, no register staging.  A key row of D
// bf16 is CH = D/8 chunks of 16 bytes; chunk c of key k sits at slot c ^ (k % CH),
// so the 32 keys an MFMA operand read touches fall on distinct banks.  K is read
// as the A operand of S^T = K Q^T (16 bytes per lane).  V is read with the gfx950
// LDS transpose load: within each 16-lane group, lane i returns element i % 4 of
// the 8-byte rows addressed by lanes i/4, i/4 + 4, i/4 + 8, i/4 + 12; addressing
// key kb + r/4, dims d0 + 4 (r % 4) from lane r hands every lane four consecutive
// keys of one dimension, which is the V^T operand of O^T = V^T P^T.
constexpr int kStages = 4;
// LDS slot of 16-byte chunk c of key k is c ^ kv_swz(k): a bijection of the low key
// bits, so 16 consecutive keys (K operand reads) hit 16 different slots, and the
// 4 consecutive keys x 2 chunks of one transpose-read group hit 8 different slots.
template <int CH>
__device__ inline int kv_swz(int key) {
  return ((((key & 3) << 1) | ((key >> 2) & 1) | (key & 8))) & (CH - 1);
}
typedef short v4s __attribute__((ext_vector_type(4)));

__device__ inline float xor32_f(float v) {  // the value of lane l ^ 32
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float((threadIdx.x & 32) ? r[0] : r[1]);
}
// Wait until at most n vector-memory operations of this wave are outstanding.
template <int n>
__device__ inline void vm_wait() {
  static_assert(n < 64, "vmcnt field");
  __builtin_amdgcn_s_waitcnt((n & 0xf) | ((n >> 4) << 14) | (0x7 << 4) | (0xf << 8));
}
__device__ inline void lds_barrier() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Eight transpose reads and the wait for them in one inline-asm block.  Written
// through the compiler's own LDS reads, the wait insertion would treat them as
// possibly aliasing the LDS tiles still being filled and wait for every
// outstanding load; inside one block the results exist only after the wait.
__device__ inline uint32_t lds_addr(const char* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}
typedef int v4i __attribute__((ext_vector_type(4)));
// Four 16-byte reads and their wait.
__device__ inline void ds_read_b128_x4(v4i (&r)[4], const uint32_t (&ad)[4]) {
  asm volatile(
      "ds_read_b128 %0, %4\n"
      "ds_read_b128 %1, %5\n"
      "ds_read_b128 %2, %6\n"
      "ds_read_b128 %3, %7\n"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3])
      : "v"(ad[0]), "v"(ad[1]), "v"(ad[2]), "v"(ad[3]));
}
// Eight independent 16-byte reads and their wait.
__device__ inline void ds_read_b128_x8(v4i (&r)[8], const uint32_t (&ad)[8]) {
  asm volatile(
      "ds_read_b128 %0, %8\n"
      "ds_read_b128 %1, %9\n"
      "ds_read_b128 %2, %10\n"
      "ds_read_b128 %3, %11\n"
      "ds_read_b128 %4, %12\n"
      "ds_read_b128 %5, %13\n"
      "ds_read_b128 %6, %14\n"
      "ds_read_b128 %7, %15\n"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]), "=&v"(r[6]), "=&v"(r[7])
      : "v"(ad[0]), "v"(ad[1]), "v"(ad[2]), "v"(ad[3]), "v"(ad[4]), "v"(ad[5]), "v"(ad[6]), "v"(ad[7]));
}
// One 4-byte and one 8-byte read and their wait.
__device__ inline int ds_read_i32(uint32_t ad) {
  int r;
  asm volatile("ds_read_b32 %0, %1\ns_waitcnt lgkmcnt(0)" : "=v"(r) : "v"(ad));
  return r;
}
__device__ inline uint64_t ds_read_u64(uint32_t ad) {
  uint64_t r;
  asm volatile("ds_read_b64 %0, %1\ns_waitcnt lgkmcnt(0)" : "=v"(r) : "v"(ad));
  return r;
}
// Eight transpose reads at ad[j] + OFF and their wait.
template <int OFF>
__device__ inline void ds_read_tr16_x8(v4s (&r)[8], const uint32_t (&ad)[8]) {
  asm volatile(
      "ds_read_b64_tr_b16 %0, %8 offset:%16\n"
      "ds_read_b64_tr_b16 %1, %9 offset:%16\n"
      "ds_read_b64_tr_b16 %2, %10 offset:%16\n"
      "ds_read_b64_tr_b16 %3, %11 offset:%16\n"
      "ds_read_b64_tr_b16 %4, %12 offset:%16\n"
      "ds_read_b64_tr_b16 %5, %13 offset:%16\n"
      "ds_read_b64_tr_b16 %6, %14 offset:%16\n"
      "ds_read_b64_tr_b16 %7, %15 offset:%16\n"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]), "=&v"(r[6]), "=&v"(r[7])
      : "v"(ad[0]), "v"(ad[1]), "v"(ad[2]), "v"(ad[3]), "v"(ad[4]), "v"(ad[5]), "v"(ad[6]), "v"(ad[7]), "n"(OFF));
}

// Eight waves: wave w owns query rows 32 (w % 4) .. + 31 of the block and key half
// w / 4 (keys 32 (w / 4) .. + 31) of every tile, so each SIMD runs two waves whose
// MFMA and VALU work interleave; the two halves of a row merge in LDS at the end.
template <int D>
__global__ __launch_bounds__(512) void attn_mfma_kernel(AttnArgs a) {
  constexpr int ROWB = D * 2;           // bytes per key row
  constexpr int CH = D / 8;             // 16-byte chunks per key row
  constexpr int TILE_B = kTile * ROWB;  // bytes per K (or V) tile
  constexpr int KPB = 1024 / ROWB;      // keys per 1 KB wave load
  constexpr int LOADS = TILE_B / 1024 / 8;  // wave loads per tile per operand
  static_assert(LOADS >= 1 && LOADS * 8 * 1024 == TILE_B, "tile split over the eight waves");
  __shared__ __attribute__((aligned(1024))) char sKV[kStages][2][TILE_B];
  __shared__ int s_page[kMaxSplitPages];
  __shared__ int s_plink[64];        // the request's parent links (parent-link mode)
  __shared__ __attribute__((aligned(16))) uint32_t s_ancin[128];  // the request's ancestor rows as 32-bit halves (row mode)

  const int tid = threadIdx.x, lane = tid & 63, wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wr = wid & 3, kh = wid >> 2;  // row block, key half
  // XCD-aware order: consecutive logical workgroups (the splits and query blocks
  // of one KV head) land on the same XCD and share its L2.
  const int W = a.batch * a.hkv * a.qblocks * a.S;
  const int per_xcd = (W + 7) / 8;
  const int L = (int)(blockIdx.x % 8) * per_xcd + (int)(blockIdx.x / 8);
  if (L >= W) return;
  int blk = L;
  const int s = blk % a.S;
  blk /= a.S;
  const int qb = blk % a.qblocks;
  blk /= a.qblocks;
  const int g = blk % a.hkv;
  const int b = blk / a.hkv;
  const int hpg = a.hq / a.hkv;
  const int G = a.n_max * hpg;

  const int k_begin = s * a.split_len;
  // the request's sizes first (scalar reads): later waits for them leave the tile
  // loads in flight
  const int n = uniform_read(a.n_nodes + b);
  const int ctx = uniform_read(a.ctx_len + b);
  const __bf16* kbase = (const __bf16*)a.k;
  const __bf16* vbase = (const __bf16*)a.v;
  // tile it -> stage it % kStages; wave w issues LOADS 1 KB loads of K and of V.
  // Keys at or past `kend` read key kend - 1 instead (valid memory; masked later).
  auto issue_tile = [&](int it, int kend, auto key_off) {
    const int t0 = k_begin + it * kTile;
    char* dk = sKV[it % kStages][0];
    char* dv = sKV[it % kStages][1];
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int kbi = wid * LOADS + i;
      const int key = kbi * KPB + lane / CH, slot = lane % CH;
      const int c = slot ^ kv_swz<CH>(key);
      const int t = min(t0 + key, kend - 1);
      const int64_t off = key_off(t) + c * 8;
      __builtin_amdgcn_global_load_lds((const void*)(kbase + off), (__attribute__((address_space(3))) void*)(dk + kbi * 1024), 16, 0, 0);
      __builtin_amdgcn_global_load_lds((const void*)(vbase + off), (__attribute__((address_space(3))) void*)(dv + kbi * 1024), 16, 0, 0);
    }
  };
  auto flat_off = [&](int t) -> int64_t { return (((int64_t)b * a.kv_capacity + t) * a.hkv + g) * D; };
  // Q and the ancestor row go out first, before the request's lengths are known: the row's
  // node index is clamped into [0, n_max) so the addresses are valid for every row,
  // and rows that turn out dead drop what they loaded
  const int r = qb * kMfmaRowsPerWg + wr * 32 + (lane & 31);
  const int node = r / hpg;
  const int node_c = min(node, a.n_max - 1);
  const int h = g * hpg + r % hpg;
  // Q, the parent links and the ancestor rows reach LDS by DMA like the K/V tiles
  // (no register loads before the loop, so no wait for a register covers the tiles
  // in flight).  Q rows of the block (row j: node j / hpg, head g hpg + j % hpg) go
  // to stage kStages - 1 in the K tiles' swizzled layout; the first tile that uses
  // that stage is issued after every wave has read its Q fragments.
  {
    constexpr int QLOADS = kMfmaRowsPerWg * ROWB / 1024 / 8;  // 1 KB loads per wave
    static_assert(QLOADS * 8 * 1024 == 2 * TILE_B, "Q fills one stage (K and V parts)");
    char* dq = sKV[kStages - 1][0];
#pragma unroll
    for (int i = 0; i < QLOADS; ++i) {
      const int kbi = wid * QLOADS + i;
      const int row = kbi * KPB + lane / CH, slot = lane % CH;
      const int rg = qb * kMfmaRowsPerWg + row;
      const int nq = min(rg / hpg, a.n_max - 1);
      const __bf16* src = (const __bf16*)a.q + (((int64_t)b * a.n_max + nq) * a.hq + g * hpg + rg % hpg) * D +
                          (slot ^ kv_swz<CH>(row)) * 8;
      __builtin_amdgcn_global_load_lds((const void*)src, (__attribute__((address_space(3))) void*)(dq + kbi * 1024), 16, 0, 0);
    }
    if (wid == 0) {
      const int64_t base = (int64_t)b * a.n_max;
      if (a.parent) {
        __builtin_amdgcn_global_load_lds((const void*)(a.parent + base + min(lane, a.n_max - 1)),
                                         (__attribute__((address_space(3))) void*)s_plink, 4, 0, 0);
      } else {
        const uint32_t* w32 = (const uint32_t*)(a.anc + base);
        __builtin_amdgcn_global_load_lds((const void*)(w32 + min(lane, 2 * a.n_max - 1)),
                                         (__attribute__((address_space(3))) void*)s_ancin, 4, 0, 0);
        __builtin_amdgcn_global_load_lds((const void*)(w32 + min(lane + 64, 2 * a.n_max - 1)),
                                         (__attribute__((address_space(3))) void*)(s_ancin + 64), 4, 0, 0);
      }
    }
  }
  bf16x8 qf[D / 16];  // Q fragments: lane holds row r, dims kk*16 + 8*(lane/32) .. +8
  // Exactly kStages - 1 tiles go out before the loop, in straight-line code, so that
  // the waits for the loads above count the tile loads issued after them and leave
  // those in flight.  Contiguous KV: they go out now, before the request's lengths
  // are known, keys clamped to the capacity (tiles past the split's end load valid
  // memory that is never used).
  constexpr int kAhead = kStages - 1;
  if (!a.block_table) {
    const int cap_end = min(k_begin + a.split_len, a.kv_capacity);  // >= 1: kv_capacity >= 1
#pragma unroll
    for (int it = 0; it < kAhead; ++it) issue_tile(it, cap_end, flat_off);
  }
  const int len = request_len_of(a, n, ctx);
  bool row_live = len >= 0 && r < G && node < n;
  const int k_end = min(k_begin + a.split_len, len < 0 ? 0 : len);
  const int n_tiles = k_end > k_begin ? (k_end - k_begin + kTile - 1) / kTile : 0;

  // page ids of this split (paged KV), one lookup per key afterwards
  int bad_page = 0;
  if (a.block_table && n_tiles > 0) {
    const int p0 = k_begin / a.page_size, p1 = (k_end - 1) / a.page_size;
    for (int i = tid; i <= p1 - p0; i += 512) {
      int pg = a.block_table[(int64_t)b * a.kv_capacity + p0 + i];
      if (pg < 0 || pg >= a.n_pages) {
        bad_page = 1;
        pg = 0;  // a valid page: the request's output is unspecified, status says why
      }
      s_page[i] = pg;
    }
    __syncthreads();
  }
  const int page0 = a.block_table ? k_begin / a.page_size : 0;
  auto key_off = [&](int t) -> int64_t {  // element offset of key t (< k_end) of head g
    if (!a.block_table) return (((int64_t)b * a.kv_capacity + t) * a.hkv + g) * D;
    // an empty split reads key 0 of page 0 (valid memory, never used)
    const int pg = n_tiles > 0 ? s_page[max(t / a.page_size - page0, 0)] : 0;
    return (((int64_t)pg * a.page_size + t % a.page_size) * a.hkv + g) * D;
  };
  // Contiguous KV, a tile wholly below k_end: a uniform tile base plus per-lane 32-bit
  // offsets that are the same for every tile.
  uint32_t loff[LOADS];
#pragma unroll
  for (int i = 0; i < LOADS; ++i) {
    const int key = (wid * LOADS + i) * KPB + lane / CH, slot = lane % CH;
    loff[i] = (uint32_t)(((int64_t)key * a.hkv * D + (slot ^ kv_swz<CH>(key)) * 8) * 2);
  }
  auto issue = [&](int it) {
    const int t0 = k_begin + it * kTile;
    if (a.block_table) {
      issue_tile(it, k_end, key_off);
    } else if (t0 + kTile <= k_end) {
      const int64_t tb = ((((int64_t)b * a.kv_capacity + t0) * a.hkv + g) * D) * 2;
      const char* kt = (const char*)kbase + tb;
      const char* vt = (const char*)vbase + tb;
      char* dk = sKV[it % kStages][0];
      char* dv = sKV[it % kStages][1];
#pragma unroll
      for (int i = 0; i < LOADS; ++i) {
        const int kbi = wid * LOADS + i;
        __builtin_amdgcn_global_load_lds((const void*)(kt + loff[i]), (__attribute__((address_space(3))) void*)(dk + kbi * 1024), 16, 0, 0);
        __builtin_amdgcn_global_load_lds((const void*)(vt + loff[i]), (__attribute__((address_space(3))) void*)(dv + kbi * 1024), 16, 0, 0);
      }
    } else {
      issue_tile(it, k_end, flat_off);
    }
  };
  if (a.block_table) {  // paged KV: the first tiles go out once the page ids are known
#pragma unroll
    for (int it = 0; it < kAhead; ++it) issue_tile(it, max(k_end, 1), key_off);
  }
  int n_issued = kAhead;  // tiles whose loads are out (perhaps past n_tiles)
  // wait until this wave's loads of tile j have landed, leaving the tiles issued
  // after it (two at most) in flight; Q, the ancestor row and the parent link were
  // issued before every tile, so they have landed too
  auto wait_tile = [&](int j) {
    const int after = n_issued - 1 - j;
    if (after >= 2) vm_wait<4 * LOADS>();
    else if (after == 1) vm_wait<2 * LOADS>();
    else vm_wait<0>();
  };
  uint64_t anc_row = 0;  // set once tile 0 and the ancestor rows are in
  f32x16 acc_o[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) acc_o[db] = f32x16{};
  // Running max and sum of the row (log2 domain, scaled scores).  The max used for
  // the exponentials is raised only when a score exceeds it by more than 8 (a factor
  // 2^8): until then the terms stay below 256 and the accumulators need no rescaling.
  float m_run = -INFINITY, l_run = 0.0f;
  const float sl2 = a.scale_log2;
  // per-lane LDS byte offsets of the operand reads within a tile, fixed for the loop
  const int g4 = lane >> 4, rr = lane & 15;
  uint32_t koff[D / 16];  // K operand of key block 0, step kk (block 1: + 32 rows)
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) {
    const int key = lane & 31, c = 2 * kk + (lane >> 5);
    koff[kk] = key * ROWB + ((c ^ kv_swz<CH>(key)) * 16);
  }
  uint32_t voff[D / 32][2];  // V^T operand of d-block db, keys +0 / +8 (k-step ks: + 16 ks rows)
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int hl = 0; hl < 2; ++hl) {
      const int key = 4 * (g4 >> 1) + (rr >> 2) + 8 * hl;
      const int d = db * 32 + 16 * (g4 & 1) + 4 * (rr & 3);
      voff[db][hl] = key * ROWB + (((d >> 3) ^ kv_swz<CH>(key)) * 16) + ((d >> 2) & 1) * 8;
    }
  // The tile loop is software-pipelined: step `it` scores tile it + 1 (the MFMAs of
  // S^T = K Q^T) while it exponentiates tile it (VALU), then accumulates tile it into
  // O^T = V^T P^T (MFMAs) while it applies tile it + 1's visibility test and running
  // max (VALU), so every wave has independent matrix and vector work in flight.  A
  // step reads K of tile it + 1 and V of tile it from LDS; with kStages = 4 two more
  // tiles are in flight meanwhile.
  constexpr int NB = (D / 32 + 3) / 4;  // batches of eight V^T reads per k-step (1 for D <= 128)
  constexpr int NDB = D / 32;
  // K operand (this wave's 32 keys of tile j)
  auto read_k = [&](int j, v4i (&kr)[D / 16]) {
    const uint32_t kb = lds_addr(sKV[j % kStages][0]) + kh * 32 * ROWB;
    uint32_t ad[D / 16];
#pragma unroll
    for (int q = 0; q < D / 16; ++q) ad[q] = kb + koff[q];
    if constexpr (D == 128) ds_read_b128_x8(kr, ad);
    else ds_read_b128_x4(kr, ad);
  };
  // V^T operands of tile j for both k-steps; k-step ks covers keys 16 ks .. 16 ks + 15
  // of the half in the order sigma(k) = 8 ((k >> 2) & 1) + 4 (k >> 3) + (k & 3) that
  // the S^T accumulator gives.  D/32 blocks x (lo, hi) reads in batches of 8 (one
  // batch covers 4 d-blocks)
  auto read_v = [&](int j, v4s (&va)[2][NB][8]) {
    const uint32_t vb = lds_addr(sKV[j % kStages][1]) + kh * 32 * ROWB;
    uint32_t vad[NB][8];
#pragma unroll
    for (int bq = 0; bq < NB; ++bq)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int db = (4 * bq + q) % NDB;
        vad[bq][2 * q] = vb + voff[db][0];
        vad[bq][2 * q + 1] = vb + voff[db][1];
      }
#pragma unroll
    for (int bq = 0; bq < NB; ++bq) {
      ds_read_tr16_x8<0>(va[0][bq], vad[bq]);
      ds_read_tr16_x8<16 * ROWB>(va[1][bq], vad[bq]);
    }
  };
  static_assert(D == 64 || D == 128, "head_dim");
  auto qk = [&](const v4i (&kr)[D / 16]) {
    f32x16 acc = f32x16{};
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      bf16x8 kf;
      __builtin_memcpy(&kf, &kr[kk], sizeof(kf));
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[kk], acc, 0, 0, 0);
    }
    return acc;
  };
  // Tile j's visibility test and the running max (lane owns row lane % 32; lane ^ 32
  // holds the other keys of the half).  kMasked: some key of the tile is a tree key
  // or lies past the request's end; the other tiles (all prompt keys, the bulk of
  // the work) skip the test.  Raw scores: the scale is applied inside the exponent.
  auto prep = [&](f32x16& sc, int j, auto masked_tag) {
    constexpr bool kMasked = decltype(masked_tag)::value;
    float tmax = -INFINITY;
    if constexpr (!kMasked) {
#pragma unroll
      for (int e = 0; e < 16; ++e) tmax = fmaxf(tmax, sc[e]);
    } else {
      const int t0 = k_begin + j * kTile;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int t = t0 + kh * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
        const int jt = t - ctx;  // tree slot
        const bool vis = t < k_end && (jt < 0 || ((anc_row >> (jt & 63)) & 1ull));
        const float v = vis ? sc[e] : -INFINITY;
        sc[e] = v;
        tmax = fmaxf(tmax, v);
      }
    }
    tmax = fmaxf(tmax, xor32_f(tmax)) * sl2;
    if (!row_live) tmax = -INFINITY;
    if (__any(tmax > m_run + 8.0f)) {  // raise the reference max (rare after the first tile)
      // (a side effect keeps this a branch: executed on every tile, the rescale
      // below would cost more than the rest of the tile's vector work)
      asm volatile("");
      const float m_new = fmaxf(m_run, tmax);
      const float alpha = (m_new == -INFINITY || m_run == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < D / 32; ++db) acc_o[db] *= alpha;
      m_run = m_new;
    }
  };
  // P of a prepared tile (bf16, the two k-steps) and its row sum
  auto expo = [&](const f32x16& sc, bf16x8 (&pf)[2]) {
    const float neg_m = m_run == -INFINITY ? 0.0f : -m_run;
    float psum = 0.0f;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const float p = __builtin_amdgcn_exp2f(fmaf(sc[e], sl2, neg_m));
      psum += p;
      pf[e >> 3][e & 7] = (__bf16)p;
    }
    psum += xor32_f(psum);
    l_run += m_run == -INFINITY ? 0.0f : psum;
  };
  auto pv = [&](const v4s (&va)[2][NB][8], const bf16x8 (&pf)[2]) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const v4s lohi[2] = {va[ks][db / 4][2 * (db % 4)], va[ks][db / 4][2 * (db % 4) + 1]};
        bf16x8 vf;
        __builtin_memcpy(&vf, lohi, sizeof(vf));
        acc_o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[ks], acc_o[db], 0, 0, 0);
      }
  };
  // tiles below min(ctx, k_end) hold prompt keys only
  const int n_plain = min(n_tiles, max(0, (min(ctx, k_end) - k_begin) / kTile));
  wait_tile(0);
  lds_barrier();  // every wave's part of tile 0 is in LDS, and Q, the links or rows
  {
    const uint32_t qb_lds = lds_addr(sKV[kStages - 1][0]) + wr * 32 * ROWB;
    v4i qr[D / 16];
    uint32_t ad[D / 16];
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) ad[kk] = qb_lds + koff[kk];
    if constexpr (D == 128) ds_read_b128_x8(qr, ad);
    else ds_read_b128_x4(qr, ad);
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) __builtin_memcpy(&qf[kk], &qr[kk], sizeof(qf[kk]));
  }
  uint64_t anc_raw;
  if (a.parent) {  // ancestor rows from the parent links, built by every wave
    const int plink = lane < a.n_max ? ds_read_i32(lds_addr((const char*)s_plink) + 4 * lane) : -1;
    bool ok;
    const uint64_t anc_l = tree_ancestors_wave(plink, n, a.n_max, &ok);
    anc_raw = shfl_u64(anc_l, node_c);
    row_live = row_live && ok;  // a request that is not a tree gets zero rows
    if (tid == 0 && !ok && len >= 0 && g == 0 && qb == 0 && s == 0) report(a.status, SPEC_ERR_BAD_TREE);
  } else {
    anc_raw = ds_read_u64(lds_addr((const char*)s_ancin) + 8 * node_c);
  }
  anc_row = row_live ? anc_raw : 0ull;
  if (!row_live)
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) qf[kk] = bf16x8{};
  f32x16 s_cur = f32x16{};  // scores of the tile being finished, prepared
  if (n_tiles > 0) {
    v4i kr[D / 16];
    read_k(0, kr);
    s_cur = qk(kr);
    if (n_plain > 0) prep(s_cur, 0, std::false_type{});
    else prep(s_cur, 0, std::true_type{});
  }
  auto step = [&](int it, auto masked_next) {
    wait_tile(it + 1);
    lds_barrier();  // tile it + 1 is in LDS; every wave is done with tile it - 1's stage
    if (it + kStages - 1 < n_tiles) {
      issue(it + kStages - 1);
      ++n_issued;
    }
    v4i kr[D / 16];
    read_k(it + 1, kr);
    v4s va[2][NB][8];
    read_v(it, va);
    const f32x16 s_next0 = qk(kr);
    bf16x8 pf[2];
    expo(s_cur, pf);
    pv(va, pf);
    f32x16 s_next = s_next0;
    prep(s_next, it + 1, masked_next);
    s_cur = s_next;
  };
  int it = 0;
  for (; it + 1 < n_plain; ++it) step(it, std::false_type{});
  for (; it + 1 < n_tiles; ++it) step(it, std::true_type{});
  if (n_tiles > 0) {  // the last tile
    v4s va[2][NB][8];
    read_v(it, va);
    bf16x8 pf[2];
    expo(s_cur, pf);
    pv(va, pf);
  }
  vm_wait<0>();  // tiles issued past the split's end have landed before LDS is reused
  if (bad_page) report(a.status, SPEC_ERR_BAD_INPUT);
  // ---- merge the two key halves of each row, split by head dimension: the
  // key-half-0 wave finishes dims [0, D/2) and the key-half-1 wave dims [D/2, D).
  // Each hands the partner the half it does not finish, with its (m, l), through
  // LDS (the K/V stages are consumed by then) ----
  constexpr int NH = D / 64;            // accumulator blocks per half of the dims
  constexpr int NV4 = NH * 16 / 4;      // float4 per lane handed over
  float4* xw = reinterpret_cast<float4*>(&sKV[0][0][0]) + (wr * 2 + kh) * (NV4 + 1) * 64;     // written here
  float4* xr = reinterpret_cast<float4*>(&sKV[0][0][0]) + (wr * 2 + 1 - kh) * (NV4 + 1) * 64; // partner's
  lds_barrier();  // every wave is done with the K/V stages
  const bool lo_half = kh == 0;  // this wave finishes dims [0, D/2)
  // (register blocks are picked with selects: the index must stay compile-time)
  {
#pragma unroll
    for (int i = 0; i < NV4; ++i) {
      const int blk = i / 4, e = 4 * (i % 4);
      xw[i * 64 + lane] = make_float4(lo_half ? acc_o[NH + blk][e] : acc_o[blk][e],
                                      lo_half ? acc_o[NH + blk][e + 1] : acc_o[blk][e + 1],
                                      lo_half ? acc_o[NH + blk][e + 2] : acc_o[blk][e + 2],
                                      lo_half ? acc_o[NH + blk][e + 3] : acc_o[blk][e + 3]);
    }
    xw[NV4 * 64 + lane] = make_float4(m_run, l_run, 0.0f, 0.0f);
  }
  lds_barrier();
  float fin[NH][16];  // the finished half of the accumulators
  {
    const float4 ml = xr[NV4 * 64 + lane];
    const float mb = ml.x, lb = ml.y;
    const float m = fmaxf(m_run, mb);
    const float wa = m_run == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m_run - m);
    const float wb = mb == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(mb - m);
    l_run = l_run * wa + lb * wb;
    m_run = m;
#pragma unroll
    for (int i = 0; i < NV4; ++i) {
      const float4 o = xr[i * 64 + lane];
      const int blk = i / 4, e = 4 * (i % 4);
      fin[blk][e] = (lo_half ? acc_o[blk][e] : acc_o[NH + blk][e]) * wa + o.x * wb;
      fin[blk][e + 1] = (lo_half ? acc_o[blk][e + 1] : acc_o[NH + blk][e + 1]) * wa + o.y * wb;
      fin[blk][e + 2] = (lo_half ? acc_o[blk][e + 2] : acc_o[NH + blk][e + 2]) * wa + o.z * wb;
      fin[blk][e + 3] = (lo_half ? acc_o[blk][e + 3] : acc_o[NH + blk][e + 3]) * wa + o.w * wb;
    }
  }
  // ---- write this split's partials (one split: the output rows themselves): the
  // wave's 32 rows x D/2 dims go through LDS (the partner's hand-over area, read by
  // now) so that they leave as whole 16-byte row pieces ----
  const bool direct = a.direct != 0;
  const int64_t n_rows = (int64_t)a.batch * a.n_max * a.hq;  // rows of one split's partials
  const bool row_out = r < G && node < a.n_max;
  const int64_t orow = ((int64_t)b * a.n_max + node) * a.hq + h;
  const int64_t prow = (int64_t)s * n_rows + orow;
  if (!direct && kh == 0 && row_out && lane < 32) {
    a.mpart[prow] = m_run;
    a.lpart[prow] = l_run;
  }
  if (direct && len < 0 && g == 0 && qb == 0 && tid == 0) report(a.status, SPEC_ERR_BAD_INPUT);
  constexpr int HB = D;               // bytes of half a row in bf16
  constexpr int OROW = HB + 16;       // bytes per staged half row (padded)
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): the hand-over reads are done
  char* so = reinterpret_cast<char*>(xr);
  {
    // an output row is zero unless its request is valid, its node exists and (rows
    // given) its ancestor row holds the node itself
    const bool keep = !direct || (row_live && ((anc_row >> (node & 63)) & 1ull));
    const float inv_l = l_run > 0.0f ? 1.0f / l_run : 0.0f;
#pragma unroll
    for (int db = 0; db < NH; ++db)
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4) {
        const int d = db * 32 + 8 * e4 + 4 * (lane >> 5);  // within the half
        bf16x4 o4;
#pragma unroll
        for (int i = 0; i < 4; ++i) o4[i] = keep ? (__bf16)(fin[db][4 * e4 + i] * inv_l) : (__bf16)0.0f;
        *reinterpret_cast<bf16x4*>(so + (lane & 31) * OROW + d * 2) = o4;
      }
  }
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's LDS writes are done
  __builtin_amdgcn_wave_barrier();
  // 16-byte pieces: lane covers piece (lane % CPR) of rows lane / CPR + rpi * j
  constexpr int CPR = HB / 16;     // pieces per half row
  constexpr int RPI = 64 / CPR;    // rows per wave instruction
#pragma unroll
  for (int j = 0; j < 32 / RPI; ++j) {
    const int rl = j * RPI + lane / CPR;  // row within the wave
    const int rg = qb * kMfmaRowsPerWg + wr * 32 + rl;
    const int nd2 = rg / hpg;
    if (rg < G && nd2 < a.n_max) {
      const int64_t orow2 = ((int64_t)b * a.n_max + nd2) * a.hq + g * hpg + rg % hpg;
      const int4 v = *reinterpret_cast<const int4*>(so + rl * OROW + (lane % CPR) * 16);
      char* dst = (direct ? (char*)a.out + orow2 * D * 2 : (char*)a.opart + ((int64_t)s * n_rows + orow2) * D * 2) +
                  kh * HB + (lane % CPR) * 16;
      *reinterpret_cast<int4*>(dst) = v;
    }
  }
}

// ---------------------------------------------------------------------------
// Shuffle path
// ---------------------------------------------------------------------------
template <int D, typename T>
__global__ __launch_bounds__(256) void attn_shfl_kernel(AttnArgs a) {
  constexpr int NV = D / 64;  // head dims per lane
  __shared__ float sQ[kShflRowsPerWg * D];
  __shared__ float sK[kTile * (D + 1)];
  __shared__ float sV[kTile * D];
  __shared__ uint64_t s_anc[64];
  __shared__ int s_tree_ok;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  int blk = blockIdx.x;
  const int s = blk % a.S;
  blk /= a.S;
  const int qb = blk % a.qblocks;
  blk /= a.qblocks;
  const int g = blk % a.hkv;
  const int b = blk / a.hkv;
  const int hpg = a.hq / a.hkv;
  const int G = a.n_max * hpg;
  const int len = request_len(a, b);
  const int n = a.n_nodes[b];
  const int ctx = a.ctx_len[b];
  const int k_begin = s * a.split_len;
  const int k_end = min(k_begin + a.split_len, len < 0 ? 0 : len);
  const T* qg = (const T*)a.q;
  const T* kg = (const T*)a.k;
  const T* vg = (const T*)a.v;

  for (int x = tid; x < kShflRowsPerWg * D; x += 256) {
    const int rr = qb * kShflRowsPerWg + x / D;
    const int node = rr / hpg, h = g * hpg + rr % hpg;
    float val = 0.0f;
    if (rr < G && node < n && len >= 0) val = (float)qg[(((int64_t)b * a.n_max + node) * a.hq + h) * D + x % D];
    sQ[x] = val;
  }
  bool tree_ok = true;
  if (a.parent) {  // ancestor rows of this request from its parent links, shared through LDS
    if (wid == 0) {
      const int p = lane < a.n_max ? a.parent[(int64_t)b * a.n_max + lane] : -1;
      bool ok;
      s_anc[lane] = tree_ancestors_wave(p, n, a.n_max, &ok);
      if (lane == 0) s_tree_ok = ok;
      if (lane == 0 && !ok && len >= 0 && g == 0 && qb == 0 && s == 0) report(a.status, SPEC_ERR_BAD_TREE);
    }
    __syncthreads();
    tree_ok = s_tree_ok;
  }
  // per-wave rows: wid, wid + 4, wid + 8, wid + 12
  float m_run[4], l_run[4], o[4][NV];
  uint64_t anc_row[4];
  bool live[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int rr = qb * kShflRowsPerWg + wid + 4 * j;
    const int node = rr / hpg;
    live[j] = len >= 0 && rr < G && node < n && tree_ok;
    anc_row[j] = live[j] ? (a.parent ? s_anc[node] : a.anc[(int64_t)b * a.n_max + node]) : 0ull;
    m_run[j] = -INFINITY;
    l_run[j] = 0.0f;
#pragma unroll
    for (int v = 0; v < NV; ++v) o[j][v] = 0.0f;
  }
  int bad_page = 0;
  for (int t0 = k_begin; t0 < k_end; t0 += kTile) {
    __syncthreads();
    for (int x = tid; x < kTile * D; x += 256) {
      const int key = x / D, d = x % D, t = t0 + key;
      float kv = 0.0f, vv = 0.0f;
      if (t < k_end) {
        const int64_t off = kv_off(a, b, t, g);
        if (off >= 0) {
          kv = (float)kg[off + d];
          vv = (float)vg[off + d];
        } else {
          bad_page = 1;
        }
      }
      sK[key * (D + 1) + d] = kv;
      sV[key * D + d] = vv;
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (!live[j]) continue;  // uniform per wave
      const int rl = wid + 4 * j;
      const int t = t0 + lane;
      float sc = 0.0f;
      for (int d = 0; d < D; ++d) sc = fmaf(sQ[rl * D + d], sK[lane * (D + 1) + d], sc);
      const bool vis = t < k_end && key_visible(t, len, ctx, anc_row[j]);
      sc = vis ? sc * a.scale_log2 : -INFINITY;
      const float tmax = wave_max_f(sc);
      const float m_new = fmaxf(m_run[j], tmax);
      if (m_new == -INFINITY) continue;
      const float alpha = __builtin_amdgcn_exp2f(m_run[j] - m_new);
      const float p = __builtin_amdgcn_exp2f(sc - m_new);
      l_run[j] = l_run[j] * alpha + wave_sum_f(p);
      m_run[j] = m_new;
#pragma unroll
      for (int v = 0; v < NV; ++v) o[j][v] *= alpha;
      for (int key = 0; key < kTile; ++key) {
        const float pk = __shfl(p, key);
#pragma unroll
        for (int v = 0; v < NV; ++v) o[j][v] = fmaf(pk, sV[key * D + lane + 64 * v], o[j][v]);
      }
    }
  }
  if (bad_page) report(a.status, SPEC_ERR_BAD_INPUT);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int rr = qb * kShflRowsPerWg + wid + 4 * j;
    if (rr >= G) continue;
    const int node = rr / hpg, h = g * hpg + rr % hpg;
    const int64_t prow = (((int64_t)s * a.batch + b) * a.n_max + node) * a.hq + h;
    if (lane == 0) {
      a.mpart[prow] = m_run[j];
      a.lpart[prow] = l_run[j];
    }
    const float inv_l = l_run[j] > 0.0f ? 1.0f / l_run[j] : 0.0f;
#pragma unroll
    for (int v = 0; v < NV; ++v) ((T*)a.opart)[prow * D + lane + 64 * v] = (T)(o[j][v] * inv_l);
  }
}

// ---------------------------------------------------------------------------
// Split combine: one wave per output row (b, node, head); the row body is shared
// with the verification step's logit pass
// ---------------------------------------------------------------------------
template <int D, typename T>
__global__ __launch_bounds__(256) void attn_combine_kernel(AttnArgs a, T* __restrict__ out) {
  attn_combine_row<D, T>(a, out, (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6));
}

struct AttnPlan {
  bool mfma;
  int S, split_len, qblocks;
};

inline AttnPlan make_plan(int32_t batch, int32_t n_max, int32_t hq, int32_t hkv, int32_t max_kv_len, int32_t dtype) {
  AttnPlan p;
  const int G = n_max * (hq / hkv);
  p.mfma = dtype == SPEC_BF16 && G >= 16;
  const int rows_per_wg = p.mfma ? kMfmaRowsPerWg : kShflRowsPerWg;
  p.qblocks = (G + rows_per_wg - 1) / rows_per_wg;
  const int tiles = max(1, (max_kv_len + kTile - 1) / kTile);
  const int64_t base = (int64_t)batch * hkv * p.qblocks;
  const int64_t target = p.mfma ? 256 : 512;  // MFMA: about one workgroup per CU
  int S = (int)std::min<int64_t>((target + base - 1) / base, tiles);
  S = std::max(S, 1);
  int tiles_per_split = (tiles + S - 1) / S;
  // a split's page ids must fit the LDS table (16-token pages or larger)
  tiles_per_split = std::min(tiles_per_split, (kMaxSplitPages - 1) * 16 / kTile);
  p.S = (tiles + tiles_per_split - 1) / tiles_per_split;
  p.split_len = tiles_per_split * kTile;
  return p;
}

inline size_t attn_ws_bytes(const AttnPlan& p, int32_t batch, int32_t n_max, int32_t hq, int32_t D) {
  const size_t rows = (size_t)p.S * batch * n_max * hq;
  return 2 * rows * sizeof(float) + rows * D * sizeof(float);  // fp32 partials for fp32 inputs
}


}  // namespace spectree

extern "C" size_t spec_tree_attention_workspace_size(int32_t batch, int32_t n_max, int32_t hq, int32_t hkv,
                                                     int32_t head_dim, int32_t max_kv_len) {
  using namespace spectree;
  if (batch < 1 || n_max < 1 || hq < 1 || hkv < 1 || hq % hkv || head_dim < 1 || max_kv_len < 1) return 0;
  // the MFMA plan has fewer splits; size for the larger of the two
  const AttnPlan p0 = make_plan(batch, n_max, hq, hkv, max_kv_len, SPEC_F32);
  const AttnPlan p1 = make_plan(batch, n_max, hq, hkv, max_kv_len, SPEC_BF16);
  return std::max(attn_ws_bytes(p0, batch, n_max, hq, head_dim), attn_ws_bytes(p1, batch, n_max, hq, head_dim));
}

namespace spectree {

// The split combine's own launch.
int attention_combine_launch(const AttnCombine& c, void* stream) {
  if (c.rows <= 0) return SPEC_OK;
  hipStream_t st = (hipStream_t)stream;
  const dim3 g2((unsigned)((c.rows + 3) / 4)), blk(256);
  if (c.dtype == SPEC_BF16) {
    if (c.head_dim == 128)
      hipLaunchKernelGGL((attn_combine_kernel<128, __bf16>), g2, blk, 0, st, c.a, (__bf16*)c.out);
    else
      hipLaunchKernelGGL((attn_combine_kernel<64, __bf16>), g2, blk, 0, st, c.a, (__bf16*)c.out);
  } else {
    if (c.head_dim == 128)
      hipLaunchKernelGGL((attn_combine_kernel<128, float>), g2, blk, 0, st, c.a, (float*)c.out);
    else
      hipLaunchKernelGGL((attn_combine_kernel<64, float>), g2, blk, 0, st, c.a, (float*)c.out);
  }
  SPEC_LAUNCH_CHECK();
  return SPEC_OK;
}

// Checks the arguments and launches the attention kernel and the split combine, with
// the split partials in `workspace` (workspace_bytes long).  With `defer`, the
// combine is not launched but described there (rows 0 when the plan needs none), for
// a later launch of the same stream to run.
int attention_launch(const void* q, const void* k, const void* v, int32_t dtype, const int32_t* block_table,
                     int32_t page_size, int32_t kv_capacity, int32_t n_pages, const int32_t* ctx_len,
                     const int32_t* n_nodes, const int32_t* parent, const uint64_t* anc_mask, int32_t batch,
                     int32_t n_max, int32_t hq, int32_t hkv, int32_t head_dim, int32_t max_kv_len, float scale,
                     void* out, void* workspace, size_t workspace_bytes, int32_t* status, void* stream,
                     AttnCombine* defer) {
  if (!q || !k || !v || !ctx_len || !n_nodes || !out) return SPEC_ERR_INVALID_ARG;
  if ((parent == nullptr) == (anc_mask == nullptr)) return SPEC_ERR_INVALID_ARG;  // exactly one of the two
  if (batch < 1 || n_max < 1 || n_max > 64 || hq < 1 || hkv < 1 || hq % hkv != 0) return SPEC_ERR_INVALID_ARG;
  if (kv_capacity < 1 || max_kv_len < 1 || !(scale > 0.0f) || isinf(scale)) return SPEC_ERR_INVALID_ARG;
  if (block_table && (page_size < 1 || n_pages < 1)) return SPEC_ERR_INVALID_ARG;
  if (head_dim != 64 && head_dim != 128) return SPEC_ERR_UNSUPPORTED;
  if (dtype != SPEC_F32 && dtype != SPEC_BF16) return SPEC_ERR_UNSUPPORTED;
  const AttnPlan p = make_plan(batch, n_max, hq, hkv, max_kv_len, dtype);
  // the MFMA path keeps a split's page ids in LDS, sized for pages of 16 tokens or more
  if (p.mfma && block_table && page_size < 16) return SPEC_ERR_UNSUPPORTED;
  if (!workspace || workspace_bytes < attn_ws_bytes(p, batch, n_max, hq, head_dim)) return SPEC_ERR_WORKSPACE;
  int64_t grid = (int64_t)batch * hkv * p.qblocks * p.S;
  if (p.mfma) grid = (grid + 7) / 8 * 8;  // whole rounds over the 8 XCDs
  if (grid > 0x7fffffffLL) return SPEC_ERR_UNSUPPORTED;
  AttnArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.block_table = block_table;
  a.page_size = page_size;
  a.kv_capacity = kv_capacity;
  a.n_pages = n_pages;
  a.ctx_len = ctx_len;
  a.n_nodes = n_nodes;
  a.parent = parent;
  a.anc = anc_mask;
  a.batch = batch;
  a.n_max = n_max;
  a.hq = hq;
  a.hkv = hkv;
  a.head_dim = head_dim;
  a.max_kv_len = max_kv_len;
  a.scale_log2 = scale * kLog2e;
  a.S = p.S;
  a.split_len = p.split_len;
  a.qblocks = p.qblocks;
  const size_t rows = (size_t)p.S * batch * n_max * hq;
  a.mpart = (float*)workspace;
  a.lpart = a.mpart + rows;
  a.opart = (void*)(a.lpart + rows);
  a.status = status;
  a.out = out;
  a.direct = p.mfma && p.S == 1;  // one split: the output directly, no combine launch
  hipStream_t st = (hipStream_t)stream;
  const dim3 g1((unsigned)grid), blk(256);
  if (p.mfma) {
    const dim3 bm(512);  // eight waves: four row blocks x two key halves
    if (head_dim == 128)
      hipLaunchKernelGGL(attn_mfma_kernel<128>, g1, bm, 0, st, a);
    else
      hipLaunchKernelGGL(attn_mfma_kernel<64>, g1, bm, 0, st, a);
  } else if (dtype == SPEC_BF16) {
    if (head_dim == 128)
      hipLaunchKernelGGL((attn_shfl_kernel<128, __bf16>), g1, blk, 0, st, a);
    else
      hipLaunchKernelGGL((attn_shfl_kernel<64, __bf16>), g1, blk, 0, st, a);
  } else {
    if (head_dim == 128)
      hipLaunchKernelGGL((attn_shfl_kernel<128, float>), g1, blk, 0, st, a);
    else
      hipLaunchKernelGGL((attn_shfl_kernel<64, float>), g1, blk, 0, st, a);
  }
  SPEC_LAUNCH_CHECK();
  const AttnCombine c{a, out, dtype, head_dim, a.direct ? 0 : (int64_t)batch * n_max * hq};
  if (defer) {
    *defer = c;
    return SPEC_OK;
  }
  return attention_combine_launch(c, stream);
}

// ---------------------------------------------------------------------------
// Library-owned split partials for spec_tree_attention_noalloc
// ---------------------------------------------------------------------------
// One array per GPU the library runs on, held until the process ends.  In host code
// `scratch` names a host-side stand-in, not device memory: its device address is
// looked up once per device with hipGetSymbolAddress and only that address is
// handed to kernels.
constexpr size_t kAttnScratchBytes = (size_t)SPEC_TREE_ATTENTION_SCRATCH_BYTES;
static __device__ __align__(256) char scratch[kAttnScratchBytes];
constexpr int kMaxDevices = 64;
static void* g_scratch_ptr[kMaxDevices];
static std::mutex g_scratch_mu;

// Device address of the current device's array (nullptr if it cannot be resolved).
static void* device_scratch() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    g_scratch_ptr[dev] = p;
  }
  return g_scratch_ptr[dev];
}

}  // namespace spectree

extern "C" int spec_tree_attention(const void* q, const void* k, const void* v, int32_t dtype,
                                   const int32_t* block_table, int32_t page_size, int32_t kv_capacity,
                                   int32_t n_pages, const int32_t* ctx_len, const int32_t* n_nodes,
                                   const int32_t* parent, const uint64_t* anc_mask, int32_t batch, int32_t n_max,
                                   int32_t hq, int32_t hkv, int32_t head_dim, int32_t max_kv_len, float scale,
                                   void* out, void* workspace, size_t workspace_bytes, int32_t* status,
                                   void* stream) {
  return spectree::attention_launch(q, k, v, dtype, block_table, page_size, kv_capacity, n_pages, ctx_len, n_nodes,
                                    parent, anc_mask, batch, n_max, hq, hkv, head_dim, max_kv_len, scale, out,
                                    workspace, workspace_bytes, status, stream, nullptr);
}

extern "C" int spec_tree_attention_noalloc(const void* q, const void* k, const void* v, int32_t dtype,
                                           const int32_t* block_table, int32_t page_size, int32_t kv_capacity,
                                           int32_t n_pages, const int32_t* ctx_len, const int32_t* n_nodes,
                                           const int32_t* parent, const uint64_t* anc_mask, int32_t batch,
                                           int32_t n_max, int32_t hq, int32_t hkv, int32_t head_dim,
                                           int32_t max_kv_len, float scale, void* out, int32_t* status,
                                           void* stream) {
  using namespace spectree;
  // the size check needs only the host-side plan: refuse before touching the device
  if (batch >= 1 && n_max >= 1 && n_max <= 64 && hq >= 1 && hkv >= 1 && hq % hkv == 0 && max_kv_len >= 1 &&
      (head_dim == 64 || head_dim == 128) && (dtype == SPEC_F32 || dtype == SPEC_BF16) &&
      attn_ws_bytes(make_plan(batch, n_max, hq, hkv, max_kv_len, dtype), batch, n_max, hq, head_dim) >
          kAttnScratchBytes)
    return SPEC_ERR_WORKSPACE;
  void* ws = device_scratch();
  if (!ws) return SPEC_ERR_HIP;
  return attention_launch(q, k, v, dtype, block_table, page_size, kv_capacity, n_pages, ctx_len, n_nodes, parent,
                          anc_mask, batch, n_max, hq, hkv, head_dim, max_kv_len, scale, out, ws, kAttnScratchBytes,
                          status, stream, nullptr);
}
