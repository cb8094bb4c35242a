// Paged MLA decode kernels for CDNA4 (gfx950).
//
// One workgroup of 4 waves runs a work item: 64 query rows (token i, head h,
// ordered i * heads + h) of one request row against one split of its keys.
// Each wave owns 16 query rows and keeps their queries (576 dims, bf16) in
// registers for the whole item. Keys stream through LDS in tiles of 32 latent
// rows: the tile's slots come from the row's page-size-1 index list (vLLM
// pull request 53001, Purpose: one row per request, one flat index list),
// each row is fetched once with 16-byte loads straight into LDS and shared by
// all 64 query rows, i.e. by all heads, since MLA has a single latent KV head.
//
// Per tile and wave:
//   S^T = K Q^T   (v_mfma_f32_16x16x32_bf16, keys are the MFMA M side, the
//                  576-dim latent the contraction): two 16-key blocks x 18
//                  k-steps; the output leaves each lane with 8 scores of one
//                  query row.
//   mask          causal on positions -- token i of a q_b-token block sits at
//                 L - q_b + i and sees keys j <= L - q_b + i (ATOM pull
//                 request 2760, Problem) -- or only the split's key range for
//                 a non-causal draft block (vLLM pull request 53001, Purpose).
//   softmax       online, base 2 (log2 e folded into the score scale); the
//                 row max is a cross-lane max over the four 16-lane groups;
//                 the running reference max only moves when a row's tile max
//                 exceeds it by more than 8 (so exp2 stays <= 256), which
//                 skips most rescales of the 128 accumulator registers.
//   O^T += V^T P^T  P^T stays in the registers it was computed in: the lane's
//                   8 scores are exactly its B operand once keys are taken in
//                   the order {4g..4g+3, 16+4g..16+4g+3} for lane group g; V^T
//                   comes from the same LDS tile (V = the first 512 latent
//                   dims, no second load) through ds_read_b64_tr_b16, read in
//                   that same key order.
// fp8 KV is fetched as fp8 (half the HBM bytes) into a staging tile and
// converted once per tile to the bf16 tile (exact: every e4m3fn value is a
// bf16 value), so the compute core is the same for all dtypes; fp8 Q is
// converted to bf16 at load. Scales are applied to the fp32 scores and to O.
//
// The epilogue writes bf16 O and the natural-log LSE when the row has one
// split, or the split's fp32 partial (O_k, LSE_k) to the workspace; the merge
// kernel then combines a row's partials by log-sum-exp ([DSV4] Tuned ASM FP8
// decode with split plans, ATOM pull request 2462, Dependencies).
//
// LDS tile layout (bf16): a "main" array of 32 rows x 1024 bytes (latent dims
// 0..511, which are also V) and a "rope" array of 32 rows x 128 bytes (dims
// 512..575). One wave-wide 16-byte direct-to-LDS load then covers exactly one
// main row, so its pool slot is wave-uniform. Within each aligned group of 8
// 16-byte chunks of a row, chunk c is stored at c ^ swz(row); the swizzle is
// applied on the global side of the load (the LDS side of a direct load is
// fixed to 64 consecutive chunks) and keeps the K reads (8 lanes, 8 keys,
// same chunk) and the transposed V reads (16 lanes, 4 keys x 32 bytes) on
// distinct banks.
#include <hip/hip_runtime.h>
#include <cstdint>
#include <type_traits>

#include "kernel_args.h"

namespace mla {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) unsigned char lds_u8;

constexpr int kDLat = 576;
constexpr int kDV = 512;
constexpr int kNT = 32;                       // keys per tile
constexpr int kMainRow = 1024;                // bf16 bytes of dims 0..511
constexpr int kRopeRow = 128;                 // bf16 bytes of dims 512..575
constexpr int kMainBytes = kNT * kMainRow;    // 32768
constexpr int kRopeBytes = kNT * kRopeRow;    // 4096
constexpr int kTileBytes = kMainBytes + kRopeBytes;   // 36864
constexpr int kF8MainRow = 512, kF8RopeRow = 64;
constexpr int kF8MainBytes = kNT * kF8MainRow;        // 16384
constexpr int kF8TileBytes = kF8MainBytes + kNT * kF8RopeRow;  // 18432
constexpr int kKSteps = kDLat / 32;           // 18 QK k-steps (16 main + 2 rope)
constexpr int kColTiles = kDV / 16;           // 32 PV column tiles
constexpr int kLdsBytes = 2 * kTileBytes;     // 73728 for either KV dtype
constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kRescaleSlack = 8.0f;

// LDS offsets. bf16 KV: two tiles, ropes first so that every immediate
// offset of a ds_read stays below 64 KB. fp8 KV: one bf16 tile and two fp8
// staging tiles (main 16 KB + rope 2 KB each).
template <bool KV_FP8> struct Layout;
template <> struct Layout<false> {
  static constexpr int rope(int buf) { return buf * kRopeBytes; }
  static constexpr int main(int buf) { return 2 * kRopeBytes + buf * kMainBytes; }
};
template <> struct Layout<true> {
  static constexpr int rope(int) { return 0; }
  static constexpr int main(int) { return kRopeBytes; }
  static constexpr int stage(int buf) { return kTileBytes + buf * kF8TileBytes; }
};

__device__ __forceinline__ int swz(int row) { return ((row & 3) << 1) | ((row >> 2) & 1); }

__device__ __forceinline__ void wait_vm_all() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// 16-byte direct-to-LDS loads (global_load_lds_dwordx4): lane l's 16 bytes
// land at LDS byte address lds_addr + 16 l. Issued as inline assembly so the
// compiler does not treat them as pending LDS writes: it would otherwise wait
// for the next tile's loads before every LDS read of the current tile. Their
// completion is awaited explicitly (wait_vm_all) before the barrier that
// publishes a tile. The compiler never uses M0 in these kernels (checked on
// the generated code), so setting it here is safe.
__device__ __forceinline__ void dma16_sbase(const void* sbase, uint32_t voff, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
               :: "s"(lds_addr), "v"(voff), "s"(sbase) : "memory");
}
__device__ __forceinline__ void dma16_vaddr(const void* vaddr, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
               :: "s"(lds_addr), "v"(vaddr) : "memory");
}

__device__ __forceinline__ uint32_t lds_addr_of(const lds_u8* p) { return (uint32_t)(uintptr_t)p; }

template <typename T> __device__ __forceinline__ T lds_load(const lds_u8* base, int off) {
  return *(const __attribute__((address_space(3))) T*)(base + off);
}
template <typename T> __device__ __forceinline__ void lds_store(lds_u8* base, int off, T v) {
  *(__attribute__((address_space(3))) T*)(base + off) = v;
}

// 4 fp8 (OCP e4m3fn) bytes -> 4 bf16, exact.
__device__ __forceinline__ bf16x4 fp8x4_to_bf16(uint32_t w) {
  bf16x2 lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false);
  bf16x2 hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true);
  return bf16x4{lo[0], lo[1], hi[0], hi[1]};
}

__device__ __forceinline__ bf16x8 cat(bf16x4 a, bf16x4 b) {
  return bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

// ---------------------------------------------------------------------------
// Tile loader (shared by the decode kernel and the gather test hook).
//
// Every lane loads the slot of key (lane & 31) of the tile; keys past the
// split's end repeat the last valid key (finite data, masked later).
__device__ __forceinline__ int load_tile_slot(const int32_t* kv_indices, int kv0, int key0, int end,
                                              int lane) {
  int key = key0 + (lane & 31);
  key = key < end ? key : end - 1;
  return kv_indices[kv0 + key];
}

// Issue one tile's direct-to-LDS loads. bf16: wave w loads main rows 4i + w
// (one 1 KB row per instruction, slot read from lane j) and rope rows 8w..8w+7.
// fp8: 16 main instructions of two rows each and 2 rope instructions, into
// the linear staging tile.
template <bool KV_FP8>
__device__ __forceinline__ void issue_tile(const unsigned char* kv, int slot_lane, lds_u8* smem,
                                           int buf, int wave, int lane) {
  const uint32_t lds0 = lds_addr_of(smem);
  if constexpr (!KV_FP8) {
    // Rows 4i + wave have swizzle (wave << 1) | (i & 1): two per-lane offsets.
    const uint32_t off_even = (uint32_t)((lane ^ (wave << 1)) << 4);
    const uint32_t off_odd = (uint32_t)((lane ^ ((wave << 1) | 1)) << 4);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int j = 4 * i + wave;
      const int slot = __builtin_amdgcn_readlane(slot_lane, j);   // wave-uniform
      const unsigned char* row = kv + (int64_t)slot * (2 * kDLat);
      dma16_sbase(row, (i & 1) ? off_odd : off_even, lds0 + Layout<false>::main(buf) + j * kMainRow);
    }
    const int j = 8 * wave + (lane >> 3);
    const int slot = __shfl(slot_lane, j, 64);
    const unsigned char* src = kv + (int64_t)slot * (2 * kDLat) + kMainRow + (((lane & 7) ^ swz(j)) << 4);
    dma16_vaddr(src, lds0 + Layout<false>::rope(buf) + wave * 1024);
  } else {
    const uint32_t stage = lds0 + Layout<true>::stage(buf);
    const uint32_t off = (uint32_t)((lane & 31) << 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int k = 4 * i + wave;                 // rows 2k (lanes 0-31) and 2k + 1
      const int slot = __shfl(slot_lane, 2 * k + (lane >> 5), 64);
      dma16_vaddr(kv + (int64_t)slot * kDLat + off, stage + k * 1024);
    }
    if (wave < 2) {
      const int j = 16 * wave + (lane >> 2);
      const int slot = __shfl(slot_lane, j, 64);
      const unsigned char* src = kv + (int64_t)slot * kDLat + kF8MainRow + ((lane & 3) << 4);
      dma16_vaddr(src, stage + kF8MainBytes + wave * 1024);
    }
  }
}

// fp8 staging tile -> the swizzled bf16 tile: a 16-byte fp8 chunk becomes two
// bf16 chunks.
__device__ __forceinline__ void convert_tile(lds_u8* smem, int buf, int tid) {
  const int stage = Layout<true>::stage(buf);
#pragma unroll 1
  for (int i = 0; i < 4; ++i) {
    const int p = i * 256 + tid;
    const int row = p >> 5, c = p & 31;
    const u32x4 w = lds_load<u32x4>(smem, stage + row * kF8MainRow + c * 16);
    const int base = Layout<true>::main(0) + row * kMainRow;
    lds_store(smem, base + (((2 * c) ^ swz(row)) << 4), cat(fp8x4_to_bf16(w[0]), fp8x4_to_bf16(w[1])));
    lds_store(smem, base + (((2 * c + 1) ^ swz(row)) << 4), cat(fp8x4_to_bf16(w[2]), fp8x4_to_bf16(w[3])));
  }
  if (tid < 128) {
    const int row = tid >> 2, c = tid & 3;
    const u32x4 w = lds_load<u32x4>(smem, stage + kF8MainBytes + row * kF8RopeRow + c * 16);
    const int base = Layout<true>::rope(0) + row * kRopeRow;
    lds_store(smem, base + (((2 * c) ^ swz(row)) << 4), cat(fp8x4_to_bf16(w[0]), fp8x4_to_bf16(w[1])));
    lds_store(smem, base + (((2 * c + 1) ^ swz(row)) << 4), cat(fp8x4_to_bf16(w[2]), fp8x4_to_bf16(w[3])));
  }
}

// Per-lane LDS byte offsets (relative to a tile's main / rope array) of the
// K fragments (A operand of S^T = K Q^T) and the transposed V fragments (A
// operand of O^T = V^T P^T). The remaining parts of each address are
// compile-time immediates.
struct LaneOffsets {
  int k_main[2];   // k-step parity 0 / 1
  int k_rope[2];
  int v[4];        // column tile c & 3
};

__device__ __forceinline__ LaneOffsets lane_offsets(int li, int lg) {
  LaneOffsets o;
  const int sk = swz(li);   // K rows 16 kt + li share the swizzle of li
#pragma unroll
  for (int par = 0; par < 2; ++par) {
    o.k_main[par] = li * kMainRow + (((4 * par + lg) ^ sk) << 4);
    o.k_rope[par] = li * kRopeRow + (((4 * par + lg) ^ sk) << 4);
  }
  // transposed V read: source lane li of group lg points at key 4 lg + li/4,
  // columns 16 c + 4 (li % 4) .. +3
  const int vrow = 4 * lg + (li >> 2);
  const int sv = swz(vrow);
  const int half = (li & 3) >> 1, inner = (li & 1) << 3;
#pragma unroll
  for (int cr = 0; cr < 4; ++cr) o.v[cr] = vrow * kMainRow + (((2 * cr + half) ^ sv) << 4) + inner;
  return o;
}

// One KV tile: QK, mask, online softmax, PV. MAIN / ROPE are the tile's LDS
// offsets (compile-time, so they fold into the instructions' offsets).
template <int MAIN, int ROPE>
__device__ __forceinline__ void compute_tile(const lds_u8* smem, const LaneOffsets& lo,
                                             const bf16x8 (&qf)[kKSteps], f32x4 (&oacc)[kColTiles],
                                             float& m_ref, float& l_part, int key_base, int end,
                                             int pos_limit, float score_c) {
  f32x4 sacc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
  for (int ks = 0; ks < kKSteps; ++ks) {
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      bf16x8 kf;
      if (ks < 16)
        kf = lds_load<bf16x8>(smem, lo.k_main[ks & 1] + MAIN + kt * 16 * kMainRow + (ks >> 1) * 128);
      else
        kf = lds_load<bf16x8>(smem, lo.k_rope[ks & 1] + ROPE + kt * 16 * kRopeRow);
      sacc[kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[ks], sacc[kt], 0, 0, 0);
    }
  }

  // key_base = split-relative index of this lane's first score's key
  float sv[8];
  float tmax = -INFINITY;
#pragma unroll
  for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int key = key_base + kt * 16 + r;
      const bool vis = key < end && key <= pos_limit;
      const float v = vis ? sacc[kt][r] * score_c : -INFINITY;
      sv[kt * 4 + r] = v;
      tmax = fmaxf(tmax, v);
    }
  }
  tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
  tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
  const bool need = tmax > m_ref + kRescaleSlack;
  if (__ballot(need)) {   // wave-uniform
    const float alpha = need ? exp2f(m_ref - tmax) : 1.0f;
    m_ref = need ? tmax : m_ref;
    l_part *= alpha;
#pragma unroll
    for (int c = 0; c < kColTiles; ++c) oacc[c] *= alpha;
  }
  const float mu = m_ref == -INFINITY ? 0.0f : m_ref;
  bf16x8 pf;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float p = exp2f(sv[e] - mu);
    l_part += p;
    pf[e] = (__bf16)p;
  }

#pragma unroll
  for (int c = 0; c < kColTiles; ++c) {
    const int imm = MAIN + (c >> 2) * 128;
    const i16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4*)(smem + lo.v[c & 3] + imm));
    const i16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4*)(smem + lo.v[c & 3] + imm + 16 * kMainRow));
    const bf16x8 vf = cat(__builtin_bit_cast(bf16x4, v0), __builtin_bit_cast(bf16x4, v1));
    oacc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf, oacc[c], 0, 0, 0);
  }
}

// ---------------------------------------------------------------------------
template <bool Q_FP8, bool KV_FP8>
__global__ __launch_bounds__(kBlockThreads, 2) void decode_kernel(DecodeArgs a) {
  __shared__ __attribute__((aligned(16))) unsigned char smem_raw[kLdsBytes];
  lds_u8* smem = (lds_u8*)smem_raw;
  using LY = Layout<KV_FP8>;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 15, lg = lane >> 4;
  const int H = a.heads;
  const unsigned char* kv = (const unsigned char*)a.kv;
  const float q_scale = a.q_scale ? *a.q_scale : 1.0f;
  const float kv_scale = a.kv_scale ? *a.kv_scale : 1.0f;
  const float score_c = a.score_scale_log2 * q_scale * kv_scale;
  const LaneOffsets lo = lane_offsets(li, lg);

  const int g = blockIdx.x;
  const int it0 = a.plan[a.off_work_indptr + g], it1 = a.plan[a.off_work_indptr + g + 1];
  for (int it = it0; it < it1; ++it) {
    const int s = a.plan[a.off_item_split + it];
    const int m = a.plan[a.off_item_m + it];
    const int b = a.plan[a.off_split_row + s];
    const int begin = a.plan[a.off_split_begin + s];
    const int end = a.plan[a.off_split_end + s];
    const int part = a.plan[a.off_split_part + s];
    const int q0 = a.qo_indptr[b], q_b = a.qo_indptr[b + 1] - q0;
    const int kv0 = a.kv_indptr[b], L = a.kv_indptr[b + 1] - kv0;
    const int M = q_b * H;
    if (m * 64 >= M) continue;   // no query row in this tile (ragged block); uniform

    const int mr = m * 64 + wave * 16 + li;
    const bool row_ok = mr < M;
    const int tok = row_ok ? mr / H : 0;
    const int head = row_ok ? mr - tok * H : 0;
    const int pos_limit = a.causal ? (L - q_b + tok) : (L - 1);

    // Queries: lane holds Q[row li][32 ks + 8 lg .. +7] for ks = 0..17 (the
    // B operand of S^T = K Q^T).
    bf16x8 qf[kKSteps];
    if (row_ok) {
      const int64_t qrow = ((int64_t)(q0 + tok) * H + head) * kDLat;
      if constexpr (!Q_FP8) {
        const bf16x8* src = (const bf16x8*)((const uint16_t*)a.q + qrow + lg * 8);
#pragma unroll
        for (int ks = 0; ks < kKSteps; ++ks) qf[ks] = src[ks * 4];
      } else {
        const u32x2* src = (const u32x2*)((const unsigned char*)a.q + qrow + lg * 8);
#pragma unroll
        for (int ks = 0; ks < kKSteps; ++ks) {
          const u32x2 w = src[ks * 4];
          qf[ks] = cat(fp8x4_to_bf16(w[0]), fp8x4_to_bf16(w[1]));
        }
      }
    } else {
#pragma unroll
      for (int ks = 0; ks < kKSteps; ++ks) qf[ks] = bf16x8{};
    }

    f32x4 oacc[kColTiles];
#pragma unroll
    for (int c = 0; c < kColTiles; ++c) oacc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_ref = -INFINITY;   // reference max (base 2) of this lane's row
    float l_part = 0.f;        // this lane's share of the row's softmax sum

    const int ntiles = (end - begin + kNT - 1) / kNT;
    if (ntiles > 0) {
      int slot_next = load_tile_slot(a.kv_indices, kv0, begin, end, lane);
      issue_tile<KV_FP8>(kv, slot_next, smem, 0, wave, lane);
      if (ntiles > 1) slot_next = load_tile_slot(a.kv_indices, kv0, begin + kNT, end, lane);

      // One tile in buffer BUF: wait for it, start the next one into the
      // other buffer, compute.
      auto step = [&](int t, auto BUF) {
        constexpr int buf = decltype(BUF)::value;
        wait_vm_all();
        __syncthreads();   // tile t landed for every wave; tile t-1 fully consumed
        if (t + 1 < ntiles) {
          issue_tile<KV_FP8>(kv, slot_next, smem, buf ^ 1, wave, lane);
          if (t + 2 < ntiles)
            slot_next = load_tile_slot(a.kv_indices, kv0, begin + (t + 2) * kNT, end, lane);
        }
        if constexpr (KV_FP8) {
          convert_tile(smem, buf, tid);
          __syncthreads();
        }
        compute_tile<LY::main(buf), LY::rope(buf)>(smem, lo, qf, oacc, m_ref, l_part,
                                                   begin + t * kNT + lg * 4, end, pos_limit,
                                                   score_c);
      };
      for (int t = 0; t < ntiles; t += 2) {
        step(t, std::integral_constant<int, 0>{});
        if (t + 1 < ntiles) step(t + 1, std::integral_constant<int, 1>{});
      }
    }

    // Epilogue.
    float l_row = l_part + __shfl_xor(l_part, 16, 64);
    l_row += __shfl_xor(l_row, 32, 64);
    if (row_ok) {
      const bool empty = !(l_row > 0.f);
      const float inv = empty ? 0.f : kv_scale / l_row;
      const float lse = empty ? -INFINITY : (m_ref + __log2f(l_row)) * kLn2;
      if (part < 0) {
        const int64_t orow = ((int64_t)(q0 + tok) * H + head);
        uint16_t* dst = a.o + orow * kDV + lg * 4;
#pragma unroll
        for (int c = 0; c < kColTiles; ++c) {
          const f32x4 v = oacc[c] * inv;
          const bf16x4 bv = {(__bf16)v[0], (__bf16)v[1], (__bf16)v[2], (__bf16)v[3]};
          *(bf16x4*)(dst + c * 16) = bv;
        }
        if (lg == 0) a.lse[orow] = lse;
      } else {
        const int64_t prow = ((int64_t)part * a.q_len_max + tok) * H + head;
        float* dst = a.ws_o + prow * kDV + lg * 4;
#pragma unroll
        for (int c = 0; c < kColTiles; ++c) *(f32x4*)(dst + c * 16) = oacc[c] * inv;
        if (lg == 0) a.ws_lse[prow] = lse;
      }
    }
    __syncthreads();   // LDS is reused by the next item
  }
}

// ---------------------------------------------------------------------------
// Split merge: one block per (request row, query token) x 4 heads; a thread
// owns 8 output columns of one head.
__global__ __launch_bounds__(kBlockThreads) void merge_kernel(MergeArgs a) {
  const int b = blockIdx.x / a.q_len_max;
  const int i = blockIdx.x - b * a.q_len_max;
  const int s0 = a.plan[a.off_split_indptr + b];
  const int n = a.plan[a.off_split_indptr + b + 1] - s0;
  if (n <= 1) return;
  const int q0 = a.qo_indptr[b];
  if (i >= a.qo_indptr[b + 1] - q0) return;
  const int h = blockIdx.y * kMergeHeadsPerBlock + (threadIdx.x >> 6);
  if (h >= a.heads) return;
  const int col = (threadIdx.x & 63) * 8;
  const int part0 = a.plan[a.off_split_part + s0];
  const int64_t stride = (int64_t)a.q_len_max * a.heads;   // partial slots are consecutive
  const int64_t base = ((int64_t)part0 * a.q_len_max + i) * a.heads + h;

  float mx = -INFINITY;
  for (int k = 0; k < n; ++k) mx = fmaxf(mx, a.ws_lse[base + k * stride]);
  const int64_t orow = (int64_t)(q0 + i) * a.heads + h;
  uint16_t* dst = a.o + orow * kDV + col;
  if (mx == -INFINITY) {
    *(u32x4*)dst = u32x4{0u, 0u, 0u, 0u};
    if ((threadIdx.x & 63) == 0) a.lse[orow] = -INFINITY;
    return;
  }
  const float kLog2e = 1.44269504088896340736f;
  float tot = 0.f;
  for (int k = 0; k < n; ++k) tot += exp2f((a.ws_lse[base + k * stride] - mx) * kLog2e);
  const float lse = mx + __log2f(tot) * kLn2;
  f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
  for (int k = 0; k < n; ++k) {
    const float lk = a.ws_lse[base + k * stride];
    if (lk == -INFINITY) continue;
    const float w = exp2f((lk - lse) * kLog2e);
    const f32x4* src = (const f32x4*)(a.ws_o + (base + k * stride) * kDV + col);
    acc0 += w * src[0];
    acc1 += w * src[1];
  }
  const bf16x8 out = {(__bf16)acc0[0], (__bf16)acc0[1], (__bf16)acc0[2], (__bf16)acc0[3],
                      (__bf16)acc1[0], (__bf16)acc1[1], (__bf16)acc1[2], (__bf16)acc1[3]};
  *(bf16x8*)dst = out;
  if ((threadIdx.x & 63) == 0) a.lse[orow] = lse;
}

// ---------------------------------------------------------------------------
// Gather test hook: one block per split; every tile goes through the decode
// kernel's loader (and fp8 conversion) into buffer 0, then is copied out of
// LDS with the swizzle undone.
template <bool KV_FP8>
__global__ __launch_bounds__(kBlockThreads) void gather_kernel(GatherArgs a) {
  __shared__ __attribute__((aligned(16))) unsigned char smem_raw[kLdsBytes];
  lds_u8* smem = (lds_u8*)smem_raw;
  using LY = Layout<KV_FP8>;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int s = blockIdx.x;
  const int b = a.plan[a.off_split_row + s];
  const int begin = a.plan[a.off_split_begin + s], end = a.plan[a.off_split_end + s];
  const int kv0 = a.kv_indptr[b];
  const int64_t dense0 = (int64_t)(kv0 - a.kv_indptr[0]);
  const unsigned char* kv = (const unsigned char*)a.kv;
  for (int key0 = begin; key0 < end; key0 += kNT) {
    const int slot = load_tile_slot(a.kv_indices, kv0, key0, end, lane);
    issue_tile<KV_FP8>(kv, slot, smem, 0, wave, lane);
    wait_vm_all();
    __syncthreads();
    if constexpr (KV_FP8) {
      convert_tile(smem, 0, tid);
      __syncthreads();
    }
    for (int p = tid; p < kNT * 72; p += kBlockThreads) {
      const int row = p / 72, chunk = p - row * 72;
      if (key0 + row < end) {
        const int off = chunk < 64 ? LY::main(0) + row * kMainRow + ((chunk ^ swz(row)) << 4)
                                   : LY::rope(0) + row * kRopeRow + (((chunk - 64) ^ swz(row)) << 4);
        const u32x4 v = lds_load<u32x4>(smem, off);
        *(u32x4*)(a.dense + (dense0 + key0 + row) * kDLat + chunk * 8) = v;
      }
    }
    __syncthreads();
  }
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, bool q_fp8, bool kv_fp8, int grid, hipStream_t st) {
  void* args[] = {(void*)&a};
  const void* fn;
  if (!q_fp8 && !kv_fp8) fn = (const void*)decode_kernel<false, false>;
  else if (!q_fp8 && kv_fp8) fn = (const void*)decode_kernel<false, true>;
  else if (q_fp8 && !kv_fp8) fn = (const void*)decode_kernel<true, false>;
  else fn = (const void*)decode_kernel<true, true>;
  return hipLaunchKernel(fn, dim3(grid), dim3(kBlockThreads), args, 0, st);
}

hipError_t launch_merge(const MergeArgs& a, int rows, int heads, int q_len_max, hipStream_t st) {
  void* args[] = {(void*)&a};
  dim3 grid(rows * q_len_max, (heads + kMergeHeadsPerBlock - 1) / kMergeHeadsPerBlock);
  return hipLaunchKernel((const void*)merge_kernel, grid, dim3(kBlockThreads), args, 0, st);
}

hipError_t launch_gather(const GatherArgs& a, bool kv_fp8, int splits, hipStream_t st) {
  void* args[] = {(void*)&a};
  const void* fn = kv_fp8 ? (const void*)gather_kernel<true> : (const void*)gather_kernel<false>;
  return hipLaunchKernel(fn, dim3(splits), dim3(kBlockThreads), args, 0, st);
}

}  // namespace mla
