// Paged MLA decode kernels for CDNA4 (gfx950).
//
// One workgroup of 8 waves per compute unit runs a work item at a time: 64
// query rows (token i, head h, ordered i * heads + h) of one request row
// against one split of its keys. Keys stream through LDS in tiles of 32 latent
// rows: the tile's slots come from the row's page-size-1 index list (vLLM pull
// request 53001, Purpose: one row per request, one flat index list); each row
// is fetched once with 16-byte loads straight into LDS and shared by all 64
// query rows, i.e. by all heads, since MLA has a single latent KV head.
//
// The waves are specialized, two per SIMD, and work one tile apart:
//   QK team   waves 0..3; wave q owns query rows 16q..16q+15 and keeps their
//             queries (576 dims, bf16) in registers. For tile t it computes
//             S^T = K Q^T on v_mfma_f32_16x16x32_bf16 (keys are the MFMA M
//             side, the 576-dim latent the contraction), applies the mask --
//             causal on positions, token i of a q_b-token block sits at
//             L - q_b + i and sees keys j <= L - q_b + i (ATOM pull request
//             2760, Problem), or only the split's range for a non-causal draft
//             block (vLLM pull request 53001, Purpose) -- and runs the online
//             softmax in base 2. It publishes P^T (bf16) and per-row rescale
//             factors in LDS. The running reference max only moves when a
//             row's tile max exceeds it by more than 8, so most tiles need no
//             rescale of the accumulators.
//   PV team   waves 4..7; wave p owns output columns 128p..128p+127 of all 64
//             rows and accumulates O^T += V^T P^T for tile t-1, V being the
//             first 512 dims of the same LDS tile (no second load), read
//             transposed with ds_read_b64_tr_b16; each V^T fragment feeds the
//             four row blocks.
// While one team waits on its softmax or its LDS reads, the other keeps the
// SIMD's matrix core busy; one barrier per tile hands P^T over. The lane
// layout of an S^T accumulator is exactly the B operand of the PV MFMA once
// the 32 keys are taken in the order {4g..4g+3, 16+4g..16+4g+3} for lane
// group g, so P never needs a register shuffle; the V^T reads use the same
// key order.
//
// fp8 KV is fetched as fp8 (half the HBM bytes) into a staging tile and
// converted once per tile to a bf16 tile (exact: every e4m3fn value is a bf16
// value), so the compute core is the same for all dtypes; fp8 Q is converted
// to bf16 at load. Scales are applied to the fp32 scores and to O.
//
// The epilogue writes bf16 O and the natural-log LSE when the row has one
// split, or the split's fp32 partial (O_k, LSE_k) to the workspace; the merge
// kernel then combines a row's partials by log-sum-exp ([DSV4] Tuned ASM FP8
// decode with split plans, ATOM pull request 2462, Dependencies).
//
// LDS tile layout (bf16): a "main" array of 32 rows x 1024 bytes (latent dims
// 0..511, which are also V) and a "rope" array of 32 rows x 128 bytes (dims
// 512..575). One wave-wide 16-byte direct-to-LDS load covers exactly one main
// row, so its pool slot is wave-uniform. The LDS has 64 four-byte banks: main
// chunk c of row r is stored at c ^ (r & 15) (inside its aligned group of 16
// chunks) and rope chunk c at c ^ ((r >> 1) & 7), which keeps the K reads (16
// lanes, 16 keys, same chunk) and the transposed V reads (16 lanes, 4 keys x 32
// bytes) on distinct banks. The swizzle is applied on the global side of each
// load (the LDS side of a direct load is fixed to consecutive 16-byte chunks).
//
// Loads run two tiles ahead. Every wave issues the same number of loads per
// tile and waits for its own with an exact vmcnt before the barrier that
// publishes the tile; the loads are inline assembly, so the compiler neither
// waits for them early nor tracks them.
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
constexpr int kWaves = kDecodeThreads / 64;   // 8
constexpr int kTeam = kWaves / 2;             // 4 waves per team
constexpr int kRowBlocks = 4;                 // 16-row blocks per work item
constexpr int kWaveCols = kDV / kTeam;        // 128 output columns per PV wave
constexpr int kWaveColTiles = kWaveCols / 16; // 8
constexpr int kBufs = 4;                      // tile buffers (bf16 KV) / staging tiles (fp8 KV)
constexpr int kAhead = 2;                     // tiles in flight
constexpr int kSlotRing = 4;                  // per-wave ring of tile slot lists
constexpr int kTilesBytes = kBufs * kTileBytes;       // 147456 for either KV dtype
constexpr int kOffP = kTilesBytes;                    // P^T [2][4 row blocks][64 lanes] bf16x8
constexpr int kOffAlpha = kOffP + 2 * kRowBlocks * 64 * 16;   // [2][64] f32 rescale factors
constexpr int kOffFlags = kOffAlpha + 2 * 64 * 4;     // [2][4] u32 "any rescale" per QK wave
constexpr int kOffL = kOffFlags + 2 * 16;             // [64] f32 row sums (epilogue)
constexpr int kOffSlots = kOffL + 64 * 4;             // [8 waves][4][32] int32
constexpr int kOffMisc = kOffSlots + kWaves * kSlotRing * kNT * 4;     // [4] u32 (merge flag)
constexpr int kSmemBytes = kOffMisc + 16;                                // 160560
constexpr int kMaxInKernelSplits = 16;
constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kRescaleSlack = 8.0f;
static_assert(kSmemBytes <= 160 * 1024, "LDS budget");

// LDS offsets of the compute tiles. bf16 KV: four tiles, ropes first, loaded
// directly. fp8 KV: two bf16 compute tiles (QK on tile t, PV on tile t-1) and
// four fp8 staging tiles (main 16 KB + rope 2 KB each) that the loads target.
template <bool KV_FP8> struct Layout;
template <> struct Layout<false> {
  static constexpr int rope(int t) { return (t % kBufs) * kRopeBytes; }
  static constexpr int main(int t) { return kBufs * kRopeBytes + (t % kBufs) * kMainBytes; }
};
template <> struct Layout<true> {
  static constexpr int rope(int t) { return (t % 2) * kRopeBytes; }
  static constexpr int main(int t) { return 2 * kRopeBytes + (t % 2) * kMainBytes; }
  static constexpr int stage(int t) { return 2 * kTileBytes + (t % kBufs) * kF8TileBytes; }
};
static_assert(Layout<true>::stage(kBufs - 1) + kF8TileBytes <= kTilesBytes, "fp8 layout");

__device__ __forceinline__ int swz_main(int row) { return row & 15; }
__device__ __forceinline__ int swz_rope(int row) { return (row >> 1) & 7; }

// 16-byte (and 4-byte) direct-to-LDS loads: lane l's data lands at LDS byte
// address lds_addr + 16 l (4 l). Inline assembly keeps them out of the
// compiler's wait-count tracking (it would otherwise wait for the next tiles'
// loads before every LDS read of the current one); completion is awaited
// explicitly with wait_vm before the barrier that publishes a tile. The
// compiler never uses M0 in these kernels (checked on the generated code), so
// setting it here is safe.
__device__ __forceinline__ void dma16_sbase(const void* sbase, uint32_t voff, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
               :: "s"(lds_addr), "v"(voff), "s"(sbase) : "memory");
}
__device__ __forceinline__ void dma16_vaddr(const void* vaddr, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
               :: "s"(lds_addr), "v"(vaddr) : "memory");
}
__device__ __forceinline__ void dma4_vaddr(const void* vaddr, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, off"
               :: "s"(lds_addr), "v"(vaddr) : "memory");
}

// Wait until at most N of this wave's vector-memory operations are in flight.
template <int N> __device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory");
}
__device__ __forceinline__ void wait_vm_all() { wait_vm<0>(); }

__device__ __forceinline__ uint32_t lds_addr_of(const lds_u8* p) { return (uint32_t)(uintptr_t)p; }

// A copy of v the compiler cannot see through: values derived from it inside
// the tile loop are recomputed there (a few VALU ops) instead of being hoisted
// out of the loop and kept live.
__device__ __forceinline__ int opaque(int v) {
  asm volatile("" : "+v"(v));
  return v;
}

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

// Reductions over the four 16-lane groups (lanes l, l ^ 16, l ^ 32, l ^ 48):
// v_permlane32_swap and v_permlane16_swap exchange halves and odd/even
// 16-lane rows between two registers, so each step is one VALU swap.
__device__ __forceinline__ float group_max(float v) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float group_sum(float v) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// ---------------------------------------------------------------------------
// Tile loader (shared by the decode kernel and the gather test hook).

// One tile's direct-to-LDS loads, spread over NW waves (the decode kernel's
// PV team, NW = 4, or all eight waves of the gather hook); every wave issues
// the same number n of load instructions, op(i) for i = 0..n-1. slot_lane:
// lane j < 32 holds the pool slot of the tile's key j.
//   bf16: op i < 32/NW loads main row j = NW i + w (one 1 KB row per
//         instruction, its slot wave-uniform); the last op loads rope rows
//         (32/NW) w .. +32/NW-1, 8 lanes per row.
//   fp8:  op i < 16/NW loads main rows 2k, 2k + 1 for k = NW i + w (two 512-byte
//         rows per instruction) into the linear staging tile; the last op
//         loads rope rows (32/NW) w .. +32/NW-1, 4 lanes per row.
template <bool KV_FP8, int NW> struct TileDma {
  static constexpr int kMainOps = (KV_FP8 ? 16 : 32) / NW;
  static constexpr int n = kMainOps + 1;
  static constexpr int kRopeRows = kNT / NW;

  static __device__ __forceinline__ void op(int i, const unsigned char* kv, int slot_lane,
                                            uint32_t lds0, int main_off, int rope_off, int w,
                                            int lane) {
    if constexpr (!KV_FP8) {
      if (i < kMainOps) {
        const int j = NW * i + w;
        const int slot = __builtin_amdgcn_readlane(slot_lane, j);   // wave-uniform
        const unsigned char* row = kv + (int64_t)slot * (2 * kDLat);
        dma16_sbase(row, (uint32_t)((lane ^ (j & 15)) << 4), lds0 + main_off + j * kMainRow);
      } else {
        const int j = kRopeRows * w + (lane >> 3);
        const int slot = __shfl(slot_lane, j & 31, 64);
        const unsigned char* src =
            kv + (int64_t)slot * (2 * kDLat) + kMainRow + (((lane & 7) ^ swz_rope(j)) << 4);
        if (lane < 8 * kRopeRows) dma16_vaddr(src, lds0 + rope_off + w * kRopeRows * kRopeRow);
      }
    } else {
      const uint32_t stage = lds0 + main_off;   // staging tile: main then rope
      if (i < kMainOps) {
        const int k = NW * i + w;                // rows 2k (lanes 0-31) and 2k + 1
        const int slot = __shfl(slot_lane, 2 * k + (lane >> 5), 64);
        dma16_vaddr(kv + (int64_t)slot * kDLat + ((lane & 31) << 4), stage + k * 1024);
      } else {
        const int j = kRopeRows * w + (lane >> 2);
        const int slot = __shfl(slot_lane, j & 31, 64);
        const unsigned char* src = kv + (int64_t)slot * kDLat + kF8MainRow + ((lane & 3) << 4);
        if (lane < 4 * kRopeRows)
          dma16_vaddr(src, stage + kF8MainBytes + w * kRopeRows * kF8RopeRow);
      }
      (void)rope_off;
    }
  }

  // All n loads of a tile at once.
  static __device__ __forceinline__ void all(const unsigned char* kv, int slot_lane, lds_u8* smem,
                                             int main_off, int rope_off, int w, int lane_in) {
    const int lane = opaque(lane_in);
#pragma unroll
    for (int i = 0; i < n; ++i) op(i, kv, slot_lane, lds_addr_of(smem), main_off, rope_off, w, lane);
  }
};

// LDS offsets a tile's loads target: bf16 tiles are loaded in place, fp8 tiles
// into their staging tile.
template <bool KV_FP8> __device__ __forceinline__ int dma_main(int t) {
  if constexpr (KV_FP8) return Layout<true>::stage(t);
  else return Layout<false>::main(t);
}
template <bool KV_FP8> __device__ __forceinline__ int dma_rope(int t) {
  if constexpr (KV_FP8) return 0;
  else return Layout<false>::rope(t);
}

// DMA the slot list of tile `tile` (32 int32, keys clamped to the split) into
// this wave's private ring entry (one load, lanes 0-31).
__device__ __forceinline__ void issue_slots(const int32_t* kv_indices, int kv0, int begin, int end,
                                            int tile, lds_u8* smem, int wave, int lane) {
  int key = begin + tile * kNT + (lane & 31);
  key = key < end ? key : end - 1;
  const uint32_t dst =
      lds_addr_of(smem) + kOffSlots + (wave * kSlotRing + (tile % kSlotRing)) * kNT * 4;
  if (lane < 32) dma4_vaddr(kv_indices + kv0 + key, dst);
}

__device__ __forceinline__ int read_slots(const lds_u8* smem, int tile, int wave, int lane) {
  return lds_load<int>(smem, kOffSlots + (wave * kSlotRing + (tile % kSlotRing)) * kNT * 4 +
                                 (lane & 31) * 4);
}

// Slot of key (lane & 31) of a tile, straight from global memory (used by the
// gather hook, which loads one tile at a time).
__device__ __forceinline__ int load_tile_slot(const int32_t* kv_indices, int kv0, int key0, int end,
                                              int lane) {
  int key = key0 + (lane & 31);
  key = key < end ? key : end - 1;
  return kv_indices[kv0 + key];
}

// fp8 staging tile -> swizzled bf16 tile (512 threads): a 16-byte fp8 chunk
// becomes two bf16 chunks.
__device__ __forceinline__ void convert_tile(lds_u8* smem, int stage, int main_off, int rope_off,
                                             int tid) {
#pragma unroll
  for (int i = 0; i < 1024 / kDecodeThreads; ++i) {
    const int p = i * kDecodeThreads + tid;
    const int row = p >> 5, c = p & 31;
    const u32x4 w = lds_load<u32x4>(smem, stage + row * kF8MainRow + c * 16);
    const int base = main_off + row * kMainRow;
    lds_store(smem, base + (((2 * c) ^ swz_main(row)) << 4),
              cat(fp8x4_to_bf16(w[0]), fp8x4_to_bf16(w[1])));
    lds_store(smem, base + (((2 * c + 1) ^ swz_main(row)) << 4),
              cat(fp8x4_to_bf16(w[2]), fp8x4_to_bf16(w[3])));
  }
  if (tid < 128) {
    const int row = tid >> 2, c = tid & 3;
    const u32x4 w = lds_load<u32x4>(smem, stage + kF8MainBytes + row * kF8RopeRow + c * 16);
    const int base = rope_off + row * kRopeRow;
    lds_store(smem, base + (((2 * c) ^ swz_rope(row)) << 4),
              cat(fp8x4_to_bf16(w[0]), fp8x4_to_bf16(w[1])));
    lds_store(smem, base + (((2 * c + 1) ^ swz_rope(row)) << 4),
              cat(fp8x4_to_bf16(w[2]), fp8x4_to_bf16(w[3])));
  }
}

// ---------------------------------------------------------------------------
// QK team: one tile.

// K rows 16 kt + li: main chunk 4 ks + lg sits at (4 ks + lg) ^ li, i.e. at
// 16 (ks >> 2) + ((4 (ks & 3) + lg) ^ li); rope chunk 4 (ks - 16) + lg at
// (4 (ks - 16) + lg) ^ ((li >> 1) & 7).
struct KOffsets {
  int main[4];
  int rope[2];
};
__device__ __forceinline__ KOffsets k_offsets(int li, int lg) {
  KOffsets o;
#pragma unroll
  for (int s = 0; s < 4; ++s) o.main[s] = li * kMainRow + (((4 * s + lg) ^ li) << 4);
#pragma unroll
  for (int s = 0; s < 2; ++s) o.rope[s] = li * kRopeRow + (((4 * s + lg) ^ swz_rope(li)) << 4);
  return o;
}

template <int MAIN, int ROPE>
__device__ __forceinline__ void qk_tile(lds_u8* smem, int q, int lane_in, int par,
                                        const bf16x8 (&qf)[kKSteps], float& m_ref, float& l_part,
                                        int key_base, int end, int pos_limit, float score_c,
                                        bool full) {
  const int lane = opaque(lane_in);
  const KOffsets ko = k_offsets(lane & 15, lane >> 4);

  // S^T: 2 key blocks x 2 independent accumulation chains (even and odd
  // k-steps), summed at the end. The K fragments of k-step pair g+2 are read
  // while pair g is multiplied (sched_barrier keeps this order; the wait-count
  // pass then waits only for the fragments actually consumed).
  f32x4 sacc[2][2];
#pragma unroll
  for (int kt = 0; kt < 2; ++kt)
#pragma unroll
    for (int c = 0; c < 2; ++c) sacc[kt][c] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto kfrag = [&](int ks, int kt) -> bf16x8 {
    if (ks < 16)
      return lds_load<bf16x8>(smem, ko.main[ks & 3] + MAIN + kt * 16 * kMainRow + (ks >> 2) * 256);
    return lds_load<bf16x8>(smem, ko.rope[ks & 1] + ROPE + kt * 16 * kRopeRow);
  };
  constexpr int kGroups = kKSteps / 2;   // 9 pairs of k-steps, 4 fragments each
  bf16x8 kbuf[3][4];
#pragma unroll
  for (int g = 0; g < 2; ++g)
#pragma unroll
    for (int f = 0; f < 4; ++f) kbuf[g][f] = kfrag(2 * g + (f >> 1), f & 1);
#pragma unroll
  for (int g = 0; g < kGroups; ++g) {
    if (g + 2 < kGroups) {
#pragma unroll
      for (int f = 0; f < 4; ++f) kbuf[(g + 2) % 3][f] = kfrag(2 * (g + 2) + (f >> 1), f & 1);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      const int ks = 2 * g + (f >> 1), kt = f & 1;
      sacc[kt][ks & 1] =
          __builtin_amdgcn_mfma_f32_16x16x32_bf16(kbuf[g % 3][f], qf[ks], sacc[kt][ks & 1], 0, 0, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  }


  // Mask and online softmax (key_base: key of this lane's first score). A
  // tile that every row of the wave sees whole (`full`, wave-uniform) skips
  // the mask.
  float sv[8];
#pragma unroll
  for (int kt = 0; kt < 2; ++kt) {
    const f32x4 s = sacc[kt][0] + sacc[kt][1];
#pragma unroll
    for (int r = 0; r < 4; ++r) sv[kt * 4 + r] = s[r] * score_c;
  }
  if (!full) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int key = key_base + (e >> 2) * 16 + (e & 3);
      sv[e] = (key < end && key <= pos_limit) ? sv[e] : -INFINITY;
    }
  }
  float tmax = fmaxf(fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3])),
                     fmaxf(fmaxf(sv[4], sv[5]), fmaxf(sv[6], sv[7])));
  tmax = group_max(tmax);
  const bool need = tmax > m_ref + kRescaleSlack;
  // v_exp_f32 directly: arguments below -126 give 0 or a denormal, which only
  // drops weights under 2^-126 of the row maximum.
  const float alpha = need ? __builtin_amdgcn_exp2f(m_ref - tmax) : 1.0f;
  m_ref = need ? tmax : m_ref;
  l_part *= alpha;
  const float mu = m_ref == -INFINITY ? 0.0f : m_ref;
  bf16x8 pf;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float p = __builtin_amdgcn_exp2f(sv[e] - mu);
    l_part += p;
    pf[e] = (__bf16)p;
  }
  // Publish P^T and the rescale factors of this wave's rows (buffer `par`).
  lds_store(smem, kOffP + ((par * kRowBlocks + q) * 64 + lane) * 16, pf);
  if (lane < 16) lds_store(smem, kOffAlpha + (par * 64 + q * 16 + lane) * 4, alpha);
  const bool any_need = __ballot(need) != 0;
  if (lane == 0) lds_store(smem, kOffFlags + (par * 4 + q) * 4, (uint32_t)any_need);
}

// ---------------------------------------------------------------------------
// PV team: one tile (its P^T and rescale factors in buffer `par`).
// issue(c) is called at the top of column tile c's step (c = 0..7): the PV
// waves spread the next tiles' loads over their MFMAs instead of queueing them
// all at once.
template <int MAIN, typename Issue>
__device__ __forceinline__ void pv_tile(const lds_u8* smem, int p, int lane_in, int par,
                                        f32x4 (&oacc)[kRowBlocks][kWaveColTiles], Issue&& issue) {
  const int lane = opaque(lane_in);
  const int li = lane & 15, lg = lane >> 4;
  const u32x4 flags = lds_load<u32x4>(smem, kOffFlags + par * 16);
  if ((flags[0] | flags[1] | flags[2] | flags[3]) != 0) {   // uniform
#pragma unroll
    for (int rb = 0; rb < kRowBlocks; ++rb) {
      const float a = lds_load<float>(smem, kOffAlpha + (par * 64 + rb * 16 + li) * 4);
#pragma unroll
      for (int c = 0; c < kWaveColTiles; ++c) oacc[rb][c] *= a;
    }
  }
  bf16x8 pall[kRowBlocks];
#pragma unroll
  for (int rb = 0; rb < kRowBlocks; ++rb)
    pall[rb] = lds_load<bf16x8>(smem, kOffP + ((par * kRowBlocks + rb) * 64 + lane) * 16);
  // Transposed V read: source lane li of group lg points at key 4 lg + li / 4,
  // columns 16 ct + 4 (li % 4) .. +3 -- chunk 2 ct + h with h = (li & 3) / 2,
  // byte (li & 1) * 8 inside it; the chunk sits at (2 ct + h) ^ (row & 15) =
  // 2 ct ^ (h ^ (row & 15)) since h is bit 0 of the chunk index. Global column
  // tile ct = 8 p + c.
  const int vrow = 4 * lg + (li >> 2);
  const int v_row = vrow * kMainRow + ((li & 1) << 3) + p * 256;
  const int v_xor = (((li & 3) >> 1) ^ swz_main(vrow)) << 4;
  auto vfrag = [&](int c) -> bf16x8 {
    const int voff = v_row + (((2 * c) << 4) ^ v_xor);
    const i16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4*)(smem + MAIN + voff));
    const i16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4*)(smem + MAIN + voff + 16 * kMainRow));
    return cat(__builtin_bit_cast(bf16x4, v0), __builtin_bit_cast(bf16x4, v1));
  };
  bf16x8 vbuf[3];
  vbuf[0] = vfrag(0);
  vbuf[1] = vfrag(1);
#pragma unroll
  for (int c = 0; c < kWaveColTiles; ++c) {
    issue(c);
    if (c + 2 < kWaveColTiles) vbuf[(c + 2) % 3] = vfrag(c + 2);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int rb = 0; rb < kRowBlocks; ++rb)
      oacc[rb][c] =
          __builtin_amdgcn_mfma_f32_16x16x32_bf16(vbuf[c % 3], pall[rb], oacc[rb][c], 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// ---------------------------------------------------------------------------
// Per-step synchronization. Only the PV team loads tiles: before the barrier
// that publishes tile t each PV wave waits for its own loads of it -- after
// them it has issued one slot-list load plus, if tile t+1 exists, that tile's
// n loads. fp8: all eight waves then convert tile t and meet again.
template <bool KV_FP8, bool PV>
__device__ __forceinline__ void step_sync(lds_u8* smem, int t, int ntiles, int tid) {
  constexpr int n = TileDma<KV_FP8, kTeam>::n;
  if constexpr (PV) {
    if (t + 1 < ntiles) wait_vm<1 + n>();
    else if (t < ntiles) wait_vm<1>();
  }
  __syncthreads();   // tile t landed; tile t-2 and P^T of tile t-2 are free
  if constexpr (KV_FP8) {
    if (t < ntiles) {
      convert_tile(smem, Layout<true>::stage(t), Layout<true>::main(t), Layout<true>::rope(t), tid);
      __syncthreads();
    }
  }
}

// In-kernel merge of one (row b, M tile m): rows m 64 .. m 64 + 63 of the
// row's block, n <= kMaxInKernelSplits fp32 partials each (consecutive
// partial slots from part0). Thread tid takes 8 (row, 8-column chunk) pairs.
__device__ __forceinline__ void merge_tile(const DecodeArgs& a, int b, int m, int M, int n, int part0,
                                           int q0, int tid) {
  const int H = a.heads;
  const int64_t stride = (int64_t)a.q_len_max * H;   // between consecutive partial slots
  const float kLog2e = 1.44269504088896340736f;
  for (int i = 0; i < 64 * 64 / kDecodeThreads; ++i) {
    const int pair = tid + i * kDecodeThreads;
    const int rr = pair >> 6, c = pair & 63;
    const int r = m * 64 + rr;
    if (r >= M) continue;
    const int tok = r / H, h = r - tok * H;
    const int64_t base = ((int64_t)part0 * a.q_len_max + tok) * H + h;
    const int64_t orow = (int64_t)(q0 + tok) * H + h;
    float lk[kMaxInKernelSplits];
    float mx = -INFINITY;
#pragma unroll
    for (int k = 0; k < kMaxInKernelSplits; ++k) {
      lk[k] = k < n ? a.ws_lse[base + k * stride] : -INFINITY;
      mx = fmaxf(mx, lk[k]);
    }
    uint16_t* dst = a.o + orow * kDV + c * 8;
    if (mx == -INFINITY) {   // no split sees a key
      *(u32x4*)dst = u32x4{0u, 0u, 0u, 0u};
      if (c == 0) a.lse[orow] = -INFINITY;
      continue;
    }
    float tot = 0.f;
#pragma unroll
    for (int k = 0; k < kMaxInKernelSplits; ++k) {
      lk[k] = lk[k] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((lk[k] - mx) * kLog2e);
      tot += lk[k];
    }
    const float inv = 1.0f / tot;
    f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < kMaxInKernelSplits; ++k) {
      if (k < n) {
        const f32x4* src = (const f32x4*)(a.ws_o + (base + k * stride) * kDV + c * 8);
        const float wk = lk[k] * inv;   // an empty split's partial is 0 and its weight 0
        acc0 += wk * src[0];
        acc1 += wk * src[1];
      }
    }
    *(bf16x8*)dst = bf16x8{(__bf16)acc0[0], (__bf16)acc0[1], (__bf16)acc0[2], (__bf16)acc0[3],
                           (__bf16)acc1[0], (__bf16)acc1[1], (__bf16)acc1[2], (__bf16)acc1[3]};
    if (c == 0) a.lse[orow] = mx + __log2f(tot) * kLn2;
  }
}

// MERGE: the variant for in-kernel-merge plans (the default variant carries
// none of that code, which would cost the hot loops registers).
template <bool Q_FP8, bool KV_FP8, bool MERGE>
__global__ __launch_bounds__(kDecodeThreads, 1) void decode_kernel(DecodeArgs a) {
  __shared__ __attribute__((aligned(16))) unsigned char smem_raw[kSmemBytes];
  lds_u8* smem = (lds_u8*)smem_raw;
  using LY = Layout<KV_FP8>;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool qk_team = wave < kTeam;
  const int li = lane & 15, lg = lane >> 4;
  const int H = a.heads;
  const unsigned char* kv = (const unsigned char*)a.kv;
  const float q_scale = a.q_scale ? *a.q_scale : 1.0f;
  const float kv_scale = a.kv_scale ? *a.kv_scale : 1.0f;
  const float score_c = a.score_scale_log2 * q_scale * kv_scale;

  const int g = blockIdx.x;
  const int it0 = a.plan[a.off_work_indptr + g], it1 = a.plan[a.off_work_indptr + g + 1];
  for (int it = it0; it < it1; ++it) {
    const int s = a.plan[a.off_item_split + it];
    const int m = a.plan[a.off_item_m + it];
    const int b = a.plan[a.off_split_row + s];
    const int part = a.plan[a.off_split_part + s];
    const int q0 = a.qo_indptr[b], q_b = a.qo_indptr[b + 1] - q0;
    const int kv0 = a.kv_indptr[b], L = a.kv_indptr[b + 1] - kv0;
    const int s0 = a.plan[a.off_split_indptr + b];
    const int nsplit = a.plan[a.off_split_indptr + b + 1] - s0;
    int begin, end;
    if (a.uniform_ranges) {   // split k of n covers [k L / n, (k + 1) L / n) of the live length
      begin = (int)((int64_t)(s - s0) * L / nsplit);
      end = (int)((int64_t)(s - s0 + 1) * L / nsplit);
    } else {
      begin = a.plan[a.off_split_begin + s];
      end = a.plan[a.off_split_end + s];
    }
    const int M = q_b * H;
    if (m * 64 >= M) continue;   // no query row in this tile (ragged block); uniform
    const int ntiles = (end - begin + kNT - 1) / kNT;

    if (qk_team) {
      // -------- QK team: rows 16 wave + li
      const int q = wave;
      const int mr = m * 64 + q * 16 + li;
      const bool row_ok = mr < M;
      const int tok = row_ok ? mr / H : 0;
      const int head = row_ok ? mr - tok * H : 0;
      // Causal mask on global positions: local key j sits at j * world + rank
      // of the row's P keys over all shards, token tok at P - q_b + tok; the
      // visible local keys are j <= (P - q_b + tok - rank) / world (one shard:
      // j <= L - q_b + tok). Rows past the end of the block are computed but
      // never written; they take the non-causal limit so that they never
      // force the masked path.
      const int P = a.kv_len_global ? a.kv_len_global[b] : L;
      const int qpos = P - q_b + tok - a.dcp_rank;
      const int causal_lim = qpos >= 0 ? qpos / a.dcp_world : -1;
      const int pos_limit = (a.causal && row_ok) ? causal_lim : (L - 1);
      // Rows are ordered token-major, so lane 0 holds the wave's smallest
      // position limit.
      const int pos_min = __builtin_amdgcn_readfirstlane(pos_limit);
      // lane holds Q[row][32 ks + 8 lg .. +7] for ks = 0..17 (B operand of S^T = K Q^T)
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
      float m_ref = -INFINITY, l_part = 0.f;

      if (ntiles > 0) {
        auto step = [&](int t, auto T4) {
          constexpr int t4 = decltype(T4)::value;   // t % 4
          step_sync<KV_FP8, false>(smem, t, ntiles, tid);
          if (t < ntiles) {
            const int last = begin + t * kNT + kNT - 1;   // last key of the tile
            qk_tile<LY::main(t4), LY::rope(t4)>(smem, q, lane, t4 & 1, qf, m_ref, l_part,
                                                begin + t * kNT + lg * 4, end, pos_limit, score_c,
                                                last < end && last <= pos_min);
          }
        };
        for (int t = 0; t <= ntiles; t += 4) {   // ntiles + 1 steps; the last one only hands over
          step(t, std::integral_constant<int, 0>{});
          if (t + 1 <= ntiles) step(t + 1, std::integral_constant<int, 1>{});
          if (t + 2 <= ntiles) step(t + 2, std::integral_constant<int, 2>{});
          if (t + 3 <= ntiles) step(t + 3, std::integral_constant<int, 3>{});
        }
      }

      // Epilogue: publish the rows' sums, write their LSE.
      const float l_row = group_sum(l_part);
      __syncthreads();
      if (lane < 16) lds_store(smem, kOffL + (q * 16 + lane) * 4, l_row);
      if (row_ok && lg == 0) {
        const float lse = l_row > 0.f ? (m_ref + __log2f(l_row)) * kLn2 : -INFINITY;
        if (part < 0) a.lse[(int64_t)(q0 + tok) * H + head] = lse;
        else a.ws_lse[((int64_t)part * a.q_len_max + tok) * H + head] = lse;
      }
      __syncthreads();
    } else {
      // -------- PV team: columns 128 p .. 128 p + 127 of all 64 rows
      const int p = wave - kTeam;
      f32x4 oacc[kRowBlocks][kWaveColTiles];
#pragma unroll
      for (int rb = 0; rb < kRowBlocks; ++rb)
#pragma unroll
        for (int c = 0; c < kWaveColTiles; ++c) oacc[rb][c] = f32x4{0.f, 0.f, 0.f, 0.f};

      if (ntiles > 0) {
        using Dma = TileDma<KV_FP8, kTeam>;
        // Prologue: slot lists of tiles 0..3, then the loads of tiles 0 and 1,
        // each preceded by one slot-list load so that every later wait count
        // has the same form.
#pragma unroll
        for (int t = 0; t < 2 * kAhead; ++t) issue_slots(a.kv_indices, kv0, begin, end, t, smem, p, lane);
        wait_vm<0>();
#pragma unroll
        for (int t = 0; t < kAhead; ++t) {
          issue_slots(a.kv_indices, kv0, begin, end, t + kAhead, smem, p, lane);
          if (t < ntiles)
            Dma::all(kv, read_slots(smem, t, p, lane), smem, dma_main<KV_FP8>(t), dma_rope<KV_FP8>(t), p, lane);
        }
        // Loads of tile t + 2 (into the buffers tile t - 2 used) and the slot
        // list of tile t + 4; at step t >= 1 they are spread over the MFMAs of
        // tile t - 1.
        auto loads = [&](int t, auto T4, int dlane) {
          constexpr int t4 = decltype(T4)::value;   // t % 4
          issue_slots(a.kv_indices, kv0, begin, end, t + 2 * kAhead, smem, p, dlane);
          const bool have = t + kAhead < ntiles;
          const int slot = have ? read_slots(smem, t + kAhead, p, dlane) : 0;
          return [=](int c) {
            if (have) {
#pragma unroll
              for (int i = 0; i < Dma::n; ++i)
                if (i * kWaveColTiles / Dma::n == c)
                  Dma::op(i, kv, slot, lds_addr_of(smem), dma_main<KV_FP8>((t4 + kAhead) % 4),
                          dma_rope<KV_FP8>((t4 + kAhead) % 4), p, dlane);
            }
          };
        };
        {  // step 0: no PV work yet
          step_sync<KV_FP8, true>(smem, 0, ntiles, tid);
          const int dlane = opaque(lane);
          auto issue = loads(0, std::integral_constant<int, 0>{}, dlane);
#pragma unroll
          for (int c = 0; c < kWaveColTiles; ++c) issue(c);
        }
        auto step = [&](int t, auto T4) {
          constexpr int t4 = decltype(T4)::value;   // t % 4; PV works on tile t - 1
          step_sync<KV_FP8, true>(smem, t, ntiles, tid);
          const int dlane = opaque(lane);
          pv_tile<LY::main((t4 + 3) % 4)>(smem, p, dlane, (t4 + 1) & 1, oacc, loads(t, T4, dlane));
        };
        for (int t = 1; t <= ntiles; t += 4) {
          step(t, std::integral_constant<int, 1>{});
          if (t + 1 <= ntiles) step(t + 1, std::integral_constant<int, 2>{});
          if (t + 2 <= ntiles) step(t + 2, std::integral_constant<int, 3>{});
          if (t + 3 <= ntiles) step(t + 3, std::integral_constant<int, 0>{});
        }
        wait_vm<0>();
      }

      // Epilogue: normalize with the rows' sums and write this wave's columns.
      __syncthreads();
      __syncthreads();
#pragma unroll
      for (int rb = 0; rb < kRowBlocks; ++rb) {
        const int r = m * 64 + rb * 16 + li;
        if (r >= M) continue;
        const float l = lds_load<float>(smem, kOffL + (rb * 16 + li) * 4);
        const float inv = l > 0.f ? kv_scale / l : 0.f;
        const int rt = r / H, rh = r - rt * H;
        const int col0 = p * kWaveCols + lg * 4;
        if (part < 0) {
          uint16_t* dst = a.o + ((int64_t)(q0 + rt) * H + rh) * kDV + col0;
#pragma unroll
          for (int c = 0; c < kWaveColTiles; ++c) {
            const f32x4 v = oacc[rb][c] * inv;
            const bf16x4 bv = {(__bf16)v[0], (__bf16)v[1], (__bf16)v[2], (__bf16)v[3]};
            *(bf16x4*)(dst + c * 16) = bv;
          }
        } else {
          float* dst = a.ws_o + (((int64_t)part * a.q_len_max + rt) * H + rh) * kDV + col0;
#pragma unroll
          for (int c = 0; c < kWaveColTiles; ++c) *(f32x4*)(dst + c * 16) = oacc[rb][c] * inv;
        }
      }
    }
    __syncthreads();   // LDS is reused by the next item

    // A split row with few splits is merged here by the last of its splits
    // to finish this M tile: every thread releases its partial stores, one
    // counts the arrival, and the last arrival reads the other splits'
    // partials after an acquire and writes the tile's O and LSE, then
    // re-zeroes the counter for the next call.
    if (MERGE && part >= 0 && nsplit <= a.inkernel_max_splits) {
      wait_vm_all();     // this thread's partial stores have reached L2
      __syncthreads();
      if (tid == 0) {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");   // one L2 write-back for the block
        const int old = __hip_atomic_fetch_add(a.counters + b * a.u + m, 1, __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT);
        lds_store(smem, kOffMisc, (uint32_t)(old == nsplit - 1));
      }
      __syncthreads();
      if (lds_load<uint32_t>(smem, kOffMisc) != 0u) {   // uniform
        if (tid == 0) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");   // invalidates for the block
        __syncthreads();
        merge_tile(a, b, m, M, nsplit, a.plan[a.off_split_part + s0], q0, tid);
        if (tid == 0) a.counters[b * a.u + m] = 0;
      }
      __syncthreads();
    }
  }
}

// ---------------------------------------------------------------------------
// Split merge: one block of four waves per (request row b, query token i,
// heads 4 j .. 4 j + 3) of a row with n > 1 splits (n <= 64). Lane k of a wave
// reads LSE_k and the wave reduces max and sum. With n <= 8 splits each wave
// merges one head, all n partials' loads in flight at once; with more, the
// four waves take every fourth split of one head at a time and add up in
// LDS. A lane owns 8 output columns.
__device__ __forceinline__ float wave_max(float v) {
  v = group_max(v);   // over lanes l, l^16, l^32, l^48
#pragma unroll
  for (int d = 8; d >= 1; d >>= 1) v = fmaxf(v, __shfl_xor(v, d, 64));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
  v = group_sum(v);
#pragma unroll
  for (int d = 8; d >= 1; d >>= 1) v += __shfl_xor(v, d, 64);
  return v;
}

// Weights of the n partials of one (token, head): lane k gets
// exp(LSE_k - LSE); returns false (and writes O = 0, LSE = -inf) when every
// split is empty.
__device__ __forceinline__ bool merge_weights(const MergeArgs& a, int64_t base, int64_t stride, int n,
                                              int lane, int64_t orow, float& wk, float& lse, bool writer) {
  const float lk = lane < n ? a.ws_lse[base + lane * stride] : -INFINITY;
  const float mx = wave_max(lk);
  if (mx == -INFINITY) {
    if (writer) {
      *(u32x4*)(a.o + orow * kDV + lane * 8) = u32x4{0u, 0u, 0u, 0u};
      if (lane == 0) a.lse[orow] = -INFINITY;
    }
    return false;
  }
  const float kLog2e = 1.44269504088896340736f;
  const float ek = lk == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((lk - mx) * kLog2e);
  const float tot = wave_sum(ek);
  wk = ek / tot;
  lse = mx + __log2f(tot) * kLn2;
  return true;
}

__device__ __forceinline__ void store_row(const MergeArgs& a, int64_t orow, int lane, f32x4 acc0, f32x4 acc1,
                                          float lse) {
  *(bf16x8*)(a.o + orow * kDV + lane * 8) =
      bf16x8{(__bf16)acc0[0], (__bf16)acc0[1], (__bf16)acc0[2], (__bf16)acc0[3],
             (__bf16)acc1[0], (__bf16)acc1[1], (__bf16)acc1[2], (__bf16)acc1[3]};
  if (lane == 0) a.lse[orow] = lse;
}

__global__ __launch_bounds__(kBlockThreads) void merge_kernel(MergeArgs a) {
  __shared__ f32x4 part[kBlockThreads / 64 - 1][64][2];
  constexpr int kW = kBlockThreads / 64;
  const int hgroups = (a.heads + kW - 1) / kW;
  const int hg = blockIdx.x % hgroups;
  const int bi = blockIdx.x / hgroups;
  const int b = bi / a.q_len_max;
  const int i = bi - b * a.q_len_max;
  const int s0 = a.plan[a.off_split_indptr + b];
  const int n = a.plan[a.off_split_indptr + b + 1] - s0;
  if (n <= a.skip_upto) return;   // unsplit, or merged in the decode kernel
  const int q0 = a.qo_indptr[b];
  if (i >= a.qo_indptr[b + 1] - q0) return;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int part0 = a.plan[a.off_split_part + s0];
  const int64_t stride = (int64_t)a.q_len_max * a.heads;   // partial slots are consecutive

  if (n <= 8) {   // one wave per head (uniform over the block: n is the row's)
    const int h = hg * kW + w;
    if (h >= a.heads) return;
    const int64_t base = ((int64_t)part0 * a.q_len_max + i) * a.heads + h;
    const int64_t orow = (int64_t)(q0 + i) * a.heads + h;
    float wk, lse;
    if (!merge_weights(a, base, stride, n, lane, orow, wk, lse, true)) return;
    const float* src = a.ws_o + base * kDV + lane * 8;
    f32x4 v[8][2];
#pragma unroll
    for (int k = 0; k < 8; ++k)
      if (k < n) {
        const f32x4* p = (const f32x4*)(src + k * stride * kDV);
        v[k][0] = p[0];
        v[k][1] = p[1];
      }
    f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < 8; ++k)
      if (k < n) {
        const float c = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wk), k));
        acc0 += c * v[k][0];   // an empty split's partial is 0 and its weight 0
        acc1 += c * v[k][1];
      }
    store_row(a, orow, lane, acc0, acc1, lse);
    return;
  }

  for (int hh = 0; hh < kW; ++hh) {   // four waves per head, one head at a time
    const int h = hg * kW + hh;
    if (h >= a.heads) break;          // uniform
    const int64_t base = ((int64_t)part0 * a.q_len_max + i) * a.heads + h;
    const int64_t orow = (int64_t)(q0 + i) * a.heads + h;
    float wk, lse;
    if (!merge_weights(a, base, stride, n, lane, orow, wk, lse, w == 0)) continue;   // uniform
    const float* src = a.ws_o + base * kDV + lane * 8;
    f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
    for (int k0 = w; k0 < n; k0 += 8 * kW) {
      f32x4 v[8][2];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int k = k0 + u * kW;
        if (k < n) {
          const f32x4* p = (const f32x4*)(src + k * stride * kDV);
          v[u][0] = p[0];
          v[u][1] = p[1];
        }
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int k = k0 + u * kW;
        if (k < n) {
          const float c = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wk), k));
          acc0 += c * v[u][0];
          acc1 += c * v[u][1];
        }
      }
    }
    if (w > 0) {
      part[w - 1][lane][0] = acc0;
      part[w - 1][lane][1] = acc1;
    }
    __syncthreads();
    if (w == 0) {
#pragma unroll
      for (int j = 0; j < kW - 1; ++j) {
        acc0 += part[j][lane][0];
        acc1 += part[j][lane][1];
      }
      store_row(a, orow, lane, acc0, acc1, lse);
    }
    __syncthreads();   // part[] is reused for the next head
  }
}

// ---------------------------------------------------------------------------
// Merge of decode-context-parallel shard outputs: one wave per (token, head)
// row; lane k < world reads LSE_k, the wave reduces max and sum, and every
// lane accumulates 8 columns of the weighted bf16 shard outputs (a shard with
// no visible key has O = 0 and weight 0).
__global__ __launch_bounds__(kBlockThreads) void shard_merge_kernel(ShardMergeArgs a) {
  const int row = blockIdx.x * (kBlockThreads / 64) + (threadIdx.x >> 6);
  if (row >= a.rows) return;
  const int lane = threadIdx.x & 63;
  const float lk = lane < a.world ? a.lse_parts[(int64_t)lane * a.rows + row] : -INFINITY;
  const float mx = wave_max(lk);
  uint16_t* dst = a.o + (int64_t)row * kDV + lane * 8;
  if (mx == -INFINITY) {   // no shard sees a key
    *(u32x4*)dst = u32x4{0u, 0u, 0u, 0u};
    if (lane == 0) a.lse[row] = -INFINITY;
    return;
  }
  const float kLog2e = 1.44269504088896340736f;
  const float ek = lk == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((lk - mx) * kLog2e);
  const float tot = wave_sum(ek);
  const float wk = ek / tot;
  f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
  for (int k = 0; k < a.world; ++k) {
    const float c = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wk), k));
    const bf16x8 v = *(const bf16x8*)(a.o_parts + ((int64_t)k * a.rows + row) * kDV + lane * 8);
    acc0 += c * f32x4{(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
    acc1 += c * f32x4{(float)v[4], (float)v[5], (float)v[6], (float)v[7]};
  }
  *(bf16x8*)dst = bf16x8{(__bf16)acc0[0], (__bf16)acc0[1], (__bf16)acc0[2], (__bf16)acc0[3],
                         (__bf16)acc1[0], (__bf16)acc1[1], (__bf16)acc1[2], (__bf16)acc1[3]};
  if (lane == 0) a.lse[row] = mx + __log2f(tot) * kLn2;
}

// Fills a buffer with zeros (the workspace's split counters); a kernel, not a
// memset, so that it may sit in a captured graph.
__global__ __launch_bounds__(256) void zero_kernel(uint32_t* p, int32_t words) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < words) p[i] = 0u;
}

// ---------------------------------------------------------------------------
// Gather test hook: one block per split; every tile goes through the decode
// kernel's loader (and fp8 conversion) into tile 0, then is copied out of LDS
// with the swizzle undone.
template <bool KV_FP8>
__global__ __launch_bounds__(kDecodeThreads) void gather_kernel(GatherArgs a) {
  __shared__ __attribute__((aligned(16))) unsigned char smem_raw[kTilesBytes];
  lds_u8* smem = (lds_u8*)smem_raw;
  using LY = Layout<KV_FP8>;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int s = blockIdx.x;
  const int b = a.plan[a.off_split_row + s];
  const int kv0 = a.kv_indptr[b];
  int begin = a.plan[a.off_split_begin + s], end = a.plan[a.off_split_end + s];
  if (a.uniform_ranges) {   // same ranges as the decode kernel
    const int s0 = a.plan[a.off_split_indptr + b];
    const int n = a.plan[a.off_split_indptr + b + 1] - s0;
    const int L = a.kv_indptr[b + 1] - kv0;
    begin = (int)((int64_t)(s - s0) * L / n);
    end = (int)((int64_t)(s - s0 + 1) * L / n);
  }
  const int64_t dense0 = (int64_t)(kv0 - a.kv_indptr[0]);
  const unsigned char* kv = (const unsigned char*)a.kv;
  for (int key0 = begin; key0 < end; key0 += kNT) {
    const int slot = load_tile_slot(a.kv_indices, kv0, key0, end, lane);
    TileDma<KV_FP8, kWaves>::all(kv, slot, smem, dma_main<KV_FP8>(0), dma_rope<KV_FP8>(0), wave, lane);
    wait_vm_all();
    __syncthreads();
    if constexpr (KV_FP8) {
      convert_tile(smem, Layout<true>::stage(0), LY::main(0), LY::rope(0), tid);
      __syncthreads();
    }
    for (int p = tid; p < kNT * 72; p += kDecodeThreads) {
      const int row = p / 72, chunk = p - row * 72;
      if (key0 + row < end) {
        const int off = chunk < 64 ? LY::main(0) + row * kMainRow + ((chunk ^ swz_main(row)) << 4)
                                   : LY::rope(0) + row * kRopeRow + (((chunk - 64) ^ swz_rope(row)) << 4);
        const u32x4 v = lds_load<u32x4>(smem, off);
        *(u32x4*)(a.dense + (dense0 + key0 + row) * kDLat + chunk * 8) = v;
      }
    }
    __syncthreads();
  }
}

}  // namespace

template <bool MERGE>
const void* decode_fn(bool q_fp8, bool kv_fp8) {
  if (!q_fp8 && !kv_fp8) return (const void*)decode_kernel<false, false, MERGE>;
  if (!q_fp8 && kv_fp8) return (const void*)decode_kernel<false, true, MERGE>;
  if (q_fp8 && !kv_fp8) return (const void*)decode_kernel<true, false, MERGE>;
  return (const void*)decode_kernel<true, true, MERGE>;
}

hipError_t launch_decode(const DecodeArgs& a, bool q_fp8, bool kv_fp8, int grid, hipStream_t st) {
  void* args[] = {(void*)&a};
  const void* fn = a.inkernel_max_splits > 1 ? decode_fn<true>(q_fp8, kv_fp8) : decode_fn<false>(q_fp8, kv_fp8);
  return hipLaunchKernel(fn, dim3(grid), dim3(kDecodeThreads), args, 0, st);
}

hipError_t launch_merge(const MergeArgs& a, int rows, int heads, int q_len_max, hipStream_t st) {
  void* args[] = {(void*)&a};
  constexpr int kW = kBlockThreads / 64;
  dim3 grid(rows * q_len_max * ((heads + kW - 1) / kW));
  return hipLaunchKernel((const void*)merge_kernel, grid, dim3(kBlockThreads), args, 0, st);
}

hipError_t launch_zero(uint32_t* p, int32_t words, hipStream_t st) {
  void* args[] = {(void*)&p, (void*)&words};
  return hipLaunchKernel((const void*)zero_kernel, dim3((words + 255) / 256), dim3(256), args, 0, st);
}

hipError_t launch_shard_merge(const ShardMergeArgs& a, hipStream_t st) {
  void* args[] = {(void*)&a};
  const int per = kBlockThreads / 64;
  return hipLaunchKernel((const void*)shard_merge_kernel, dim3((a.rows + per - 1) / per),
                         dim3(kBlockThreads), args, 0, st);
}

hipError_t launch_gather(const GatherArgs& a, bool kv_fp8, int splits, hipStream_t st) {
  void* args[] = {(void*)&a};
  const void* fn = kv_fp8 ? (const void*)gather_kernel<true> : (const void*)gather_kernel<false>;
  return hipLaunchKernel(fn, dim3(splits), dim3(kDecodeThreads), args, 0, st);
}

}  // namespace mla
