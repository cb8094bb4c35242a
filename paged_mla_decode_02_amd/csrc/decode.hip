// Paged MLA decode kernel for CDNA4 (gfx950), and the gather test hook that
// runs its tile loader.
//
// One workgroup of four waves (one per SIMD) runs a work item at a time: 128
// query rows (token i, head h, ordered i * heads + h) of one request row
// against one split of its keys. Keys stream through LDS in tiles of 32
// latent rows: the tile's slots come from the row's page-size-1 index list
// (vLLM pull request 53001, Purpose: one row per request, one flat index
// list); each latent row is fetched once with 16-byte loads straight into LDS
// and serves all 128 query rows, i.e. all heads, since MLA has a single latent
// KV head.
//
// Every wave does all three stages of the attention:
//   QK        wave w owns query rows 32w..32w+31 and keeps their queries (576
//             dims) in registers, staged at the head of each item through LDS
//             by the tile loader. For tile t it computes S^T = K Q^T (keys
//             are the MFMA M side, the 576-dim latent the contraction): on
//             v_mfma_f32_32x32x16_bf16 for bf16 KV, on the fp8
//             v_mfma_f32_32x32x64_f8f6f4 for fp8 KV (fp8 Q as is; bf16 Q
//             split exactly into two fp8 operands per row).
//   softmax   the mask -- causal on positions: token i of a q_b-token block
//             sits at L - q_b + i and sees keys j <= L - q_b + i (ATOM pull
//             request 2760, Problem); non-causal: only the split's range (vLLM
//             pull request 53001, Purpose) -- and the exponentials in base 2
//             against a per-row reference max, fixed at the row's first
//             visible tile, so the accumulated O is never rescaled (a tile
//             that would overflow the reference makes the item run again
//             with each row's true max). The wave publishes P^T of its rows in
//             LDS.
//   PV        wave w owns output columns 128w..128w+127 of all 128 rows and
//             accumulates O^T += V^T P^T, V being the first 512 dims of the
//             same LDS tile (no second load), read transposed with
//             ds_read_b64_tr_b16; each V^T fragment feeds the four 32-row
//             blocks.
// A wave holds 32 query rows, so every 1 KB K fragment it reads from LDS feeds
// a 32x32x16 MFMA. The lane layout of an S^T accumulator is exactly the B
// operand of the PV MFMA once the keys of a 16-key half are taken in the order
// {4g..4g+3, 8+4g..8+4g+3} for lane half g, so P never needs a register
// shuffle; the V^T reads use the same key order.
//
// The stages form a software pipeline of one step per tile, in two phases
// split by the step's only barrier: phase A of step t runs the 36 QK
// products of tile t with the softmax of tile t-1 spread between them (VALU
// work beside the matrix core) and publishes P^T(t-1); phase B runs the 32
// PV products of tile t-1 with the loads of tile t+2 spread between them,
// and the wave goes straight on to the next step's phase A.
//
// fp8 KV stays fp8 in LDS (half the HBM and LDS bytes). K fragments feed the
// fp8 QK products as they are; V^T fragments are converted to bf16 in
// registers for the bf16 PV products (exact: every e4m3fn value is a bf16
// value). Scales are applied to the fp32 scores and to O.
//
// The epilogue writes bf16 O and the natural-log LSE when the row has one
// split, or the split's normalized bf16 partial O and fp32 LSE_k to the
// workspace; the merge kernel then combines a row's partials by log-sum-exp
// ([DSV4] Tuned ASM FP8 decode with split plans, ATOM pull request 2462,
// Dependencies).
//
// LDS tile layout (bf16): a "main" array of 32 rows x 1024 bytes (latent dims
// 0..511, which are also V) and a "rope" array of 32 rows x 128 bytes (dims
// 512..575). One wave-wide 16-byte direct-to-LDS load covers exactly one main
// row, so its pool slot is wave-uniform. Rows are 1 KB apart, so every row
// starts in bank 0: main chunk c (16 bytes) of key row i is stored at
// c ^ s(i) inside its aligned group of 16 chunks, s(i) = 4 (i & 3) +
// ((i >> 2) & 3), and rope chunk c at c ^ ((i >> 1) & 7). s is a bijection
// on 0..15, so a K fragment read (16 keys per 16-lane group, one chunk each)
// covers all banks; it also moves the two low row bits into the chunk's
// 64-byte sector, so the four keys of one transposed V read land in four
// different sectors. The swizzle is applied on the global side of each load
// (the LDS side of a direct load is fixed to consecutive 16-byte chunks).
//
// Loads run two tiles ahead: step t issues tile t+2's loads, and every wave
// waits for its own loads of tile t+1 before step t's barrier, after which
// tile t+1 is visible to all waves. Waves may thus be up to one phase apart
// between two barriers; every LDS buffer is rewritten only after a barrier
// that every reader of its previous contents has passed. The loads are
// inline assembly, so the compiler neither waits for them early nor tracks
// them.
#include <hip/hip_runtime.h>
#include <cstdint>
#include <type_traits>

#include "device_common.h"
#include "kernel_args.h"

namespace mla {
namespace {

using namespace dev;

constexpr int kDLat = 576;
constexpr int kDV = 512;
constexpr int kNT = 32;                       // keys per tile
constexpr int kMainRow = 1024;                // bf16 bytes of dims 0..511
constexpr int kRopeRow = 128;                 // bf16 bytes of dims 512..575
constexpr int kMainBytes = kNT * kMainRow;    // 32768
constexpr int kRopeBytes = kNT * kRopeRow;    // 4096
constexpr int kF8MainRow = 512, kF8RopeRow = 64;
constexpr int kF8MainBytes = kNT * kF8MainRow;        // 16384
// fp8 rope: each wave's 8 rows (512 bytes) sit at the start of a 1 KB slot;
// its load runs on all 64 lanes (lanes 32-63 repeat lanes 0-31's sources
// into the slot's second half), so no lane mask splits the pipeline code.
constexpr int kF8RopeBytes = (kDecodeThreads / 64) * 1024;   // 4096
constexpr int kKSteps = kDLat / 16;           // 36 QK k-steps (32 main + 4 rope)
constexpr int kKSteps8 = kDLat / 64;          // 9 fp8 QK products (8 main + 1 rope) for fp8 Q and KV
constexpr int kWaves = kDecodeThreads / 64;   // 4
constexpr int kRows = 128;                    // query rows per work item
constexpr int kRowBlocks = kRows / 32;        // 4 blocks of 32 rows (one per wave)
constexpr int kWaveCols = kDV / kWaves;       // 128 output columns per wave
constexpr int kColTiles = kWaveCols / 32;     // 4
constexpr int kSlotRing = 4;                  // per-wave ring of tile slot lists
constexpr int kPBytes = kRowBlocks * 2 * 64 * 16;     // P^T of one tile: [4 row blocks][2 key halves][64 lanes] bf16x8
// Main tiles t-1 (PV), t (QK), t+1, t+2 (loads in flight) and rope tiles t,
// t+1, t+2, in the KV dtype (fp8 tiles are half the size).
constexpr int kMainBufs = 4, kRopeBufs = 3;
constexpr int kTilesEnd = 143360;             // end of the tile region for either KV dtype
static_assert(kMainBufs * kMainBytes + kRopeBufs * kRopeBytes <= kTilesEnd, "bf16 tiles");
static_assert(kMainBufs * kF8MainBytes + kRopeBufs * kF8RopeBytes <= kTilesEnd, "fp8 tiles");
constexpr int kOffP = kTilesEnd;                      // [2] P^T buffers (tiles of even / odd index)
constexpr int kOffL = kOffP + 2 * kPBytes;            // [128] f32 row sums (epilogue)
constexpr int kOffSlots = kOffL + kRows * 4;          // [4 waves][4][32] int32
constexpr int kOffMisc = kOffSlots + kWaves * kSlotRing * kNT * 4;     // [4] u32 (restart, merge flags)
constexpr int kOffP8Scale = kOffMisc + 16;   // fp8 PV: [4 tile parities][32 rows] u32 of scale codes
constexpr int kSmemBytes = kOffP8Scale + 4 * 32 * 4;                     // 162832
constexpr int kMaxInKernelSplits = 16;
constexpr float kRefSlack = 64.0f;       // base-2 headroom above a row's reference max
static_assert(kSmemBytes <= 160 * 1024, "LDS budget");
static_assert(kRows == 128, "the plan's M unit");
static_assert(kRows * kDV * 2 <= kTilesEnd, "epilogue staging of the item's 128 bf16 rows");

// fp8 PV (fp8 KV only): tiles t-2 and t-1 stay in LDS until the step that
// multiplies both, so the main tiles take a longer ring; P^T goes through LDS
// in fp8, [tile mod 4][4 row blocks][64 lanes] x 16 bytes (four tiles: a
// tile's P^T is read up to one step after it is written, while the waves
// may be a phase apart), with the per-(row, tile) power-of-two scales at
// kOffP8Scale, [tile mod 4][32 rows] x 4 bytes (byte rb for row block rb).
// With split bf16 queries the hi and lo operands of the last kQLds QK
// products (dims 448..575) wait in LDS after the tiles, [4 waves][2 kQLds
// links][64 lanes] x 32 bytes, instead of in 32 registers; 6 main tiles
// suffice (t-2 .. t+2 are in use during step t).
constexpr int kMainBufs8 = 6;
constexpr int kQLds = 2;
constexpr int kOffQ8 = kMainBufs8 * kF8MainBytes + kRopeBufs * kF8RopeBytes;
static_assert(kOffQ8 + kWaves * 2 * kQLds * 64 * 32 <= kTilesEnd, "fp8-PV tiles and the staged queries");
constexpr int kP8Bytes = kRowBlocks * 64 * 16;                  // 4096 per tile
static_assert(kOffP + 4 * kP8Bytes <= kOffL, "fp8 P^T of four tiles fits the P^T region");

// Query staging: at the head of a work item its 128 query rows pass through
// LDS as four 32-row tiles (tile q: the rows of wave q) in the tile layout of
// the query dtype, loaded by the tile loader with the block's row index in
// place of a pool slot. Each load instruction then moves whole rows (one
// 1 KB row, or eight 128-byte rope rows) instead of 32 bytes of 32 rows, and
// the rows reach the registers with conflict-free LDS reads. The region
// overlaps the first tiles and the P^T buffers, which the item uses only
// after its queries are in registers.
template <bool QF8> struct QStage;
template <> struct QStage<false> {
  static __device__ __forceinline__ int main(int q) { return q * kMainBytes; }
  static __device__ __forceinline__ int rope(int q) { return 4 * kMainBytes + q * kRopeBytes; }
};
template <> struct QStage<true> {
  static __device__ __forceinline__ int main(int q) { return q * kF8MainBytes; }
  static __device__ __forceinline__ int rope(int q) { return 4 * kF8MainBytes + q * kF8RopeBytes; }
};
static_assert(kWaves * (kMainBytes + kRopeBytes) <= kOffL, "bf16 query staging below the row sums");
// fp8 queries with fp8 KV (bf16 PV products): the staging region fits above
// the tile ring (it overlaps only the P^T buffers, first written in step 1),
// so tiles 0 and 1 load while the queries land.
constexpr int kOffQAbove = kMainBufs * kF8MainBytes + kRopeBufs * kF8RopeBytes;
struct QStageAbove {
  static __device__ __forceinline__ int main(int q) { return kOffQAbove + QStage<true>::main(q); }
  static __device__ __forceinline__ int rope(int q) { return kOffQAbove + QStage<true>::rope(q); }
};
static_assert(kOffQAbove + kWaves * (kF8MainBytes + kF8RopeBytes) <= kOffL, "fp8 query staging above the tiles");

// LDS offsets of tile t's buffers.
template <bool KV_FP8, bool PV8 = false> struct Layout;
template <> struct Layout<false, false> {
  static __device__ __forceinline__ int main(int t) { return (t & 3) * kMainBytes; }
  static __device__ __forceinline__ int rope(int t) { return kMainBufs * kMainBytes + (t % 3) * kRopeBytes; }
};
template <> struct Layout<true, false> {
  static __device__ __forceinline__ int main(int t) { return (t & 3) * kF8MainBytes; }
  static __device__ __forceinline__ int rope(int t) { return kMainBufs * kF8MainBytes + (t % 3) * kF8RopeBytes; }
};
template <> struct Layout<true, true> {
  static __device__ __forceinline__ int main(int t) { return (t % kMainBufs8) * kF8MainBytes; }
  static __device__ __forceinline__ int rope(int t) { return kMainBufs8 * kF8MainBytes + (t % 3) * kF8RopeBytes; }
};
__device__ __forceinline__ int p_buf(int t) { return kOffP + (t & 1) * kPBytes; }

__device__ __forceinline__ int swz_main(int row) { return ((row & 3) << 2) | ((row >> 2) & 3); }
__device__ __forceinline__ int swz_rope(int row) { return (row >> 1) & 7; }
// fp8 tiles: main rows are 512 bytes (32 chunks), rope rows 64 bytes (4
// chunks). swz_f8 is a bijection on 0..15 (a K read of 16 keys covers all
// banks) whose value >> 1 differs across the 8 keys of one transposed V read
// (4g..4g+3 and 8+4g..8+4g+3 of a 16-key half), so those 8 keys' two chunks
// land in 16 different chunk slots.
__device__ __forceinline__ int swz_f8(int row) {
  return ((row & 3) << 2) | (((row >> 3) & 1) << 1) | ((row >> 2) & 1);
}
__device__ __forceinline__ int swz_f8_rope(int row) { return (row >> 2) & 3; }

// Read-only launch metadata (plan words, indptrs, per-row lengths): nothing
// writes it during a launch, so it is read through the constant address
// space, which lets the compiler use scalar loads for uniform indices. Vector
// loads would be ordered behind the previous work item's O stores (stores
// count in the vector-memory counter), so each item's dependent chain of
// metadata reads would first wait for those stores to be acknowledged.
__device__ __forceinline__ int32_t ldc(const int32_t* p, int64_t i) {
  return ((const __attribute__((address_space(4))) int32_t*)p)[i];
}

// ---------------------------------------------------------------------------
// Tile loader (shared by the decode kernel and the gather test hook).

// One tile's direct-to-LDS loads, spread over the four waves; every wave
// issues the same number n of load instructions, op(i) for i = 0..n-1.
// The source addresses come from a TileSrc, built once per tile from the
// slot list (slot_lane: lane j < 32 holds the pool slot of the tile's key j),
// so the address arithmetic of the n loads is not a chain in front of each.
//   bf16: op i < 8 loads main row j = 4 i + w (one 1 KB row per instruction,
//         its address wave-uniform: read from lane j of the per-lane row
//         addresses); op 8 loads rope rows 8w .. 8w+7, 8 lanes per row.
//   fp8:  op i < 4 loads main rows 2k, 2k + 1 for k = 4 i + w (two 512-byte
//         rows per instruction); op 4 loads rope rows 8w .. 8w+7, 4 lanes per
//         row, into the wave's 1 KB rope slot.
template <bool KV_FP8> struct TileSrc;
template <> struct TileSrc<false> {
  uint32_t lo, hi;            // lane j < 32: byte address of key j's latent row
  const unsigned char* rope;  // this lane's source of the rope load
};
template <> struct TileSrc<true> {
  int slot_lane;
};

template <bool KV_FP8> struct TileDma {
  static constexpr int kMainOps = (KV_FP8 ? 16 : 32) / kWaves;
  static constexpr int n = kMainOps + 1;
  static constexpr int kRopeRows = kNT / kWaves;

  // Slots beyond the pool are clamped to its last row, so that no load
  // leaves the pool whatever the slot lists hold.
  static __device__ __forceinline__ TileSrc<KV_FP8> src(const unsigned char* kv, int slot_in, uint32_t max_slot,
                                                        int w, int lane) {
    const int slot_lane = (int)min((uint32_t)slot_in, max_slot);
    TileSrc<KV_FP8> t;
    if constexpr (!KV_FP8) {
      const uint64_t row = (uint64_t)(uintptr_t)kv + (uint64_t)(uint32_t)slot_lane * (2 * kDLat);
      t.lo = (uint32_t)row;
      t.hi = (uint32_t)(row >> 32);
      const int j = kRopeRows * w + (lane >> 3);
      const int slot = bpermute(j & 31, slot_lane);
      t.rope = kv + (int64_t)(uint32_t)slot * (2 * kDLat) + kMainRow + (((lane & 7) ^ swz_rope(j)) << 4);
    } else {
      t.slot_lane = slot_lane;
    }
    return t;
  }

  static __device__ __forceinline__ void op(int i, const unsigned char* kv, const TileSrc<KV_FP8>& src,
                                            uint32_t lds0, int main_off, int rope_off, int w,
                                            int lane) {
    if constexpr (!KV_FP8) {
      if (i < kMainOps) {
        const int j = kWaves * i + w;
        const uint64_t lo = (uint32_t)__builtin_amdgcn_readlane((int)src.lo, j);   // wave-uniform
        const uint64_t hi = (uint32_t)__builtin_amdgcn_readlane((int)src.hi, j);
        const unsigned char* row = (const unsigned char*)(uintptr_t)((hi << 32) | lo);
        dma16_sbase(row, (uint32_t)((lane ^ swz_main(j)) << 4), lds0 + main_off + j * kMainRow);
      } else {
        dma16_vaddr(src.rope, lds0 + rope_off + w * kRopeRows * kRopeRow);
      }
    } else {
      const int slot_lane = src.slot_lane;
      if (i < kMainOps) {
        const int k = kWaves * i + w;            // rows 2k (lanes 0-31) and 2k + 1
        const int row = 2 * k + (lane >> 5);
        const int slot = bpermute(row, slot_lane);
        dma16_vaddr(kv + (int64_t)slot * kDLat + (((lane & 31) ^ swz_f8(row)) << 4),
                    lds0 + main_off + k * 2 * kF8MainRow);
      } else {
        const int j = kRopeRows * w + ((lane & 31) >> 2);
        const int slot = bpermute(j, slot_lane);
        dma16_vaddr(kv + (int64_t)slot * kDLat + kF8MainRow + (((lane & 3) ^ swz_f8_rope(j)) << 4),
                    lds0 + rope_off + w * 1024);
      }
    }
  }

  // All n loads of a tile at once.
  static __device__ __forceinline__ void all(const unsigned char* kv, int slot_lane, uint32_t max_slot,
                                             lds_u8* smem, int main_off, int rope_off, int w, int lane_in) {
    const int lane = opaque(lane_in);
    const TileSrc<KV_FP8> s = src(kv, slot_lane, max_slot, w, lane);
#pragma unroll
    for (int i = 0; i < n; ++i) op(i, kv, s, lds_addr_of(smem), main_off, rope_off, w, lane);
  }
};

// LDS offsets a tile's loads target.
template <bool KV_FP8> __device__ __forceinline__ int dma_main(int t) { return Layout<KV_FP8>::main(t); }
template <bool KV_FP8> __device__ __forceinline__ int dma_rope(int t) { return Layout<KV_FP8>::rope(t); }

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


// ---------------------------------------------------------------------------
// QK MFMAs. They go through inline assembly so that their accumulators are
// VGPRs: the compiler gives every MFMA of a kernel the same accumulator
// class, and the AGPRs are all taken by the PV accumulators. The 36 products
// of a tile form one accumulation chain, and a product whose srcC is exactly
// the previous product's result may issue right behind it (the matrix core
// forwards the accumulator); padding between two links with wait states
// costs about 30 cycles per product, so only the last link of a chain waits
// inside its own statement until its result can be read by the VALU (12 wait
// states for v_mfma_f32_32x32x16_bf16). The compiler does not know when an
// assembly MFMA's result arrives, so nothing else may read or write the
// accumulator between two links: the library build checks the generated code
// for that. The destination of a multi-pass MFMA may not overlap its A or B
// operand, hence the early clobber on the first product of a chain (in the
// others the accumulator is an input too, so it cannot share registers with
// them).
__device__ __forceinline__ void mfma_qk_first(f32x16& d, bf16x8 a, bf16x8 b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_qk(f32x16& d, bf16x8 a, bf16x8 b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "v"(b));
}
// The last link writes its own output operand: the chain's accumulator is
// then only an input, so the compiler never needs to move it between links to
// place the result.
__device__ __forceinline__ void mfma_qk_last(f32x16& out, const f32x16& acc, bf16x8 a, bf16x8 b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %3\n\ts_nop 7\n\ts_nop 3"
               : "=&v"(out) : "v"(a), "v"(b), "v"(acc));
}

// fp8 Q with fp8 KV: the QK products take both operands in fp8
// (v_mfma_f32_32x32x64_f8f6f4, OCP e4m3 by default), so K is never converted.
// A product is 16 passes: the last link waits 22 wait states before its
// result is read. Each operand register of lane l holds 32 bytes of its row
// (key l & 31 in A, query row l & 31 in B): product p takes dims
// 64 p + 16 h .. +15 and 64 p + 32 + 16 h .. +15 (h = l >> 5) for both. The
// products sum over every dim exactly once whatever order the matrix core
// gives the 64 k positions, since A and B put the same dim in the same
// (lane half, byte) position; the exact fp8 products are accumulated in fp32
// as in the bf16 path.
__device__ __forceinline__ void mfma8_qk_first(f32x16& d, u32x8 a, u32x8 b) {
  asm volatile("v_mfma_f32_32x32x64_f8f6f4 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma8_qk(f32x16& d, u32x8 a, u32x8 b) {
  asm volatile("v_mfma_f32_32x32x64_f8f6f4 %0, %1, %2, %0" : "+v"(d) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma8_qk_last(f32x16& out, const f32x16& acc, u32x8 a, u32x8 b) {
  asm volatile("v_mfma_f32_32x32x64_f8f6f4 %0, %1, %2, %3\n\ts_nop 7\n\ts_nop 7\n\ts_nop 5"
               : "=&v"(out) : "v"(a), "v"(b), "v"(acc));
}
__device__ __forceinline__ u32x8 cat8(u32x4 a, u32x4 b) {
  return u32x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

// bf16 Q with fp8 KV takes the same fp8 products twice: every query row is
// split as x 2^A = hi + lo with hi = fp8(x 2^A) and lo = fp8(x 2^A - hi),
// A per row so that its largest |x| 2^A lies in [128, 256). hi keeps the top
// 4 significant bits of an element, lo the next 4, so the pair is exact for
// every bf16 element above 2^-2 after scaling (lo is then at least the
// smallest subnormal step 2^-9); a smaller element loses at most 2^-10, i.e.
// 2^-17 of the row's largest. The scores come out times 2^A, which the
// softmax takes out with its score scale.
__device__ __forceinline__ uint32_t pack_fp8x4(float a, float b, float c, float d) {
  const uint32_t w = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, (int)__float_as_uint(a), false);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, d, (int)w, true);
}
// bf16 elements in packed pairs -> fp8 hi and lo. hi comes straight from the
// packed bf16 pairs: v_cvt_scalef32_pk_fp8_bf16 rounds x / inv = x 2^A to
// e4m3 (nearest even), which a host model of the instruction confirmed;
// lo = fp8(x 2^A - hi), the product x 2^A being exact.
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
typedef short i16x2v __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
// In place: q[2 p] and q[2 p + 1] hold the 32 bf16 elements of product p
// (dims 64 p + 16 h .. +15, then 64 p + 32 + 16 h .. +15) and become its hi
// and lo fp8 operands. The row's largest |x| is taken over both lane halves
// (lanes l and l ^ 32 hold one row). Returns 2^-A.
__device__ __forceinline__ float split_q_rows(u32x8 (&q)[2 * kKSteps8]) {
  // largest |x| as bf16 bits (the order of non-negative floats), two per
  // dword with packed 16-bit max
  typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
  u16x2 m2 = {0, 0};
#pragma unroll
  for (int n = 0; n < 2 * kKSteps8; ++n)
#pragma unroll
    for (int d = 0; d < 8; ++d) m2 = __builtin_elementwise_max(m2, __builtin_bit_cast(u16x2, q[n][d] & 0x7FFF7FFFu));
  const uint32_t m = max((uint32_t)m2[0], (uint32_t)m2[1]);
  const float amax = half_max(__uint_as_float(m << 16));
  int ex = 0;
  if (amax > 0.f && __builtin_isfinite(amax)) frexpf(amax, &ex);   // amax in [2^(ex-1), 2^ex)
  ex = max(ex, -100);   // keeps 2^(8 - ex) and the score scale normal floats
  const float scale = ldexpf(1.0f, 8 - ex), inv = ldexpf(1.0f, ex - 8);
  // (2^A, 0) and (0, 2^A) as bf16 pairs (2^A is exact in bf16)
  const uint32_t sc_bits = __float_as_uint(scale) >> 16;
  const bf16x2v sc_lo = __builtin_bit_cast(bf16x2v, sc_bits), sc_hi = __builtin_bit_cast(bf16x2v, sc_bits << 16);
#pragma unroll
  for (int p = 0; p < kKSteps8; ++p) {
    // Stage by stage over the product's 16 dwords (scheduling barriers
    // between the stages), so that the dependent conversions of different
    // dwords interleave instead of running as one chain per dword pair.
    uint32_t w[16], hi[8], lo[8];
#pragma unroll
    for (int d = 0; d < 8; ++d) { w[d] = q[2 * p][d]; w[8 + d] = q[2 * p + 1][d]; }
    i16x2v ha[8];
#pragma unroll
    for (int k = 0; k < 8; ++k)
      ha[k] = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(__builtin_bit_cast(i16x2v, w[2 * k]), __builtin_bit_cast(bf16x2v, w[2 * k]), inv, false);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int k = 0; k < 8; ++k)
      hi[k] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(ha[k], __builtin_bit_cast(bf16x2v, w[2 * k + 1]), inv, true));
    __builtin_amdgcn_sched_barrier(0);
    float r[32];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      // -hi from the sign-flipped codes; x 2^A - hi as one bf16 dot product
      // per element against (2^A, 0) or (0, 2^A), accumulating -hi (exact:
      // the product is exact and the residual fits in a float)
      const uint32_t nh = hi[k] ^ 0x80808080u;
      const auto f01 = __builtin_amdgcn_cvt_pk_f32_fp8((int)nh, false);
      const auto f23 = __builtin_amdgcn_cvt_pk_f32_fp8((int)nh, true);
      const bf16x2v a0 = __builtin_bit_cast(bf16x2v, w[2 * k]), a1 = __builtin_bit_cast(bf16x2v, w[2 * k + 1]);
      r[4 * k] = __builtin_amdgcn_fdot2_f32_bf16(a0, sc_lo, f01[0], false);
      r[4 * k + 1] = __builtin_amdgcn_fdot2_f32_bf16(a0, sc_hi, f01[1], false);
      r[4 * k + 2] = __builtin_amdgcn_fdot2_f32_bf16(a1, sc_lo, f23[0], false);
      r[4 * k + 3] = __builtin_amdgcn_fdot2_f32_bf16(a1, sc_hi, f23[1], false);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int k = 0; k < 8; ++k) lo[k] = pack_fp8x4(r[4 * k], r[4 * k + 1], r[4 * k + 2], r[4 * k + 3]);
    q[2 * p] = u32x8{hi[0], hi[1], hi[2], hi[3], hi[4], hi[5], hi[6], hi[7]};
    q[2 * p + 1] = u32x8{lo[0], lo[1], lo[2], lo[3], lo[4], lo[5], lo[6], lo[7]};
    __builtin_amdgcn_sched_barrier(0);
  }
  return ldexpf(1.0f, ex - 8);
}

// Per-lane LDS addressing, fixed for a work item.
//   K fragment (A operand of S^T = K Q^T), k-step ks: lane l holds key
//   i = l & 31, dims 16 ks + 8 (l >> 5) .. +7 -- main chunk 2 ks + h of row i,
//   stored at (2 ks) ^ xm with xm = h ^ swz_main(i), or rope chunk
//   2 (ks - 32) + h at (2 (ks - 32)) ^ xr.
//   V^T fragment (A operand of O^T += V^T P^T), column tile ct, key half kk:
//   lane l takes column 32 (4w + ct) + (l & 31) and keys 16 kk + {4g..4g+3,
//   8+4g..8+4g+3}, g = l >> 5, as two transposed reads q = 0, 1. In each,
//   source lane li = l & 15 of a 16-lane block points at key
//   16 kk + 8 q + kb (kb = 4 g + li / 4) and columns 4 (li % 4) .. +3 of the
//   block's 16: logical chunk 16 w + 4 ct + c0 (c0 = 2 ((l >> 4) & 1) + (li & 3) / 2)
//   of that key, stored at chunk 16 w + ((4 ct + c0) ^ swz_main(8 q + kb)) =
//   16 w + 4 (ct ^ r) + (c0 ^ (2 q + g)) with r = li >> 2: the four keys of a
//   half-wave's read sit in the four different 64-byte bank sectors, and its
//   32 lanes cover all 64 banks once.
//
// fp8 tiles (K read as fp8 QK operands; V^T converted in registers, exactly):
//   K: pair j covers dims 32 j .. 32 j + 31 and lane l reads 16 bytes, dims
//   32 j + 16 h .. +15 (h = l >> 5), of key i = l & 31; pairs 2 p and 2 p + 1
//   form the A operand of fp8 product p (Q is loaded in the same order). Main chunk 2 j + h of
//   row i is stored at (2 j) ^ xm, xm = h ^ swz_f8(i); rope chunk
//   2 (j - 16) + h at (2 (j - 16)) ^ xr, xr = h ^ swz_f8_rope(i), rope row i
//   at (i / 8) 1024 + (i % 8) 64.
//   V^T: one transposed 8-bit read per fragment (ds_read_b64_tr_b8: in a
//   16-lane block, source lane s gives row s / 2 and bytes 8 (s & 1) .. +7 of
//   the block's 16 columns; result lane c gets column c of the 8 rows). Block
//   b = (l >> 4) & 3 takes columns 16 (b & 1) .. +15 of the column tile and
//   the lane-half-g keys (g = b >> 1), row r = s / 2 being key 4 g + r
//   (r < 4) or 8 + 4 g + r - 4: the key order of the P^T fragments. Column
//   chunk 8 w + 2 ct + (b & 1) of key k is stored at that ^ swz_f8(k), so
//   va = k 512 + 256 (w >> 1) + 16 ((8 (w & 1) + (b & 1)) ^ swz_f8(k)) +
//   8 (s & 1), and column tile ct flips bits 5-6.
struct LaneAddr {
  int krow, xm, rrow, xr;   // K
  int va;                   // V: bf16 kb * 1024 + 256 w + 64 r + 16 (c0 ^ g) + 8 (li & 1); fp8 as above
  int pl;                   // P: lane * 16
  int w;
};
template <bool KV_FP8> __device__ __forceinline__ LaneAddr lane_addr(int lane, int w) {
  LaneAddr a;
  const int i = lane & 31, h = lane >> 5;
  if constexpr (!KV_FP8) {
    a.krow = i * kMainRow;
    a.xm = h ^ swz_main(i);
    a.rrow = i * kRopeRow;
    a.xr = h ^ swz_rope(i);
    const int li = lane & 15, g16 = (lane >> 4) & 1, g = lane >> 5;
    const int kb = 4 * g + (li >> 2), c0 = 2 * g16 + ((li & 3) >> 1);
    a.va = kb * kMainRow + 256 * w + 64 * (li >> 2) + 16 * (c0 ^ g) + 8 * (li & 1);
  } else {
    a.krow = i * kF8MainRow;
    a.xm = h ^ swz_f8(i);
    a.rrow = (i >> 3) * 1024 + (i & 7) * kF8RopeRow;
    a.xr = h ^ swz_f8_rope(i);
    const int sl = lane & 15, b1 = (lane >> 4) & 1, g = lane >> 5, r = sl >> 1;
    const int key = r < 4 ? 4 * g + r : 8 + 4 * g + (r - 4);
    a.va = key * kF8MainRow + 256 * (w >> 1) + 16 * ((8 * (w & 1) + b1) ^ swz_f8(key)) + 8 * (sl & 1);
  }
  a.pl = lane * 16;
  a.w = w;
  return a;
}

__device__ __forceinline__ bf16x8 k_frag(const lds_u8* smem, const LaneAddr& la, int kmain, int krope, int ks) {
  if (ks < 32)
    return lds_load<bf16x8>(smem, kmain + la.krow + (ks >> 3) * 256 + (((2 * (ks & 7)) ^ la.xm) << 4));
  return lds_load<bf16x8>(smem, krope + la.rrow + (((2 * (ks - 32)) ^ la.xr) << 4));
}

// fp8 K pair j (k-steps 2 j and 2 j + 1), 16 bytes.
__device__ __forceinline__ u32x4 k_pair_f8(const lds_u8* smem, const LaneAddr& la, int kmain, int krope, int j) {
  if (j < 16) return lds_load<u32x4>(smem, kmain + la.krow + (((2 * j) ^ la.xm) << 4));
  return lds_load<u32x4>(smem, krope + la.rrow + (((2 * (j - 16)) ^ la.xr) << 4));
}
// fp8 A operand of QK product p: pairs 2 p and 2 p + 1 (dims 64 p + 16 h and
// 64 p + 32 + 16 h, 16 bytes each).
__device__ __forceinline__ u32x8 k_prod_f8(const lds_u8* smem, const LaneAddr& la, int kmain, int krope, int p) {
  return cat8(k_pair_f8(smem, la, kmain, krope, 2 * p), k_pair_f8(smem, la, kmain, krope, 2 * p + 1));
}
// Staged bf16 query row i = lane & 31, read for the split into fp8 operands:
// operand n holds 16-byte chunks 4 n + 2 h and 4 n + 2 h + 1 (dims
// 32 n + 16 h .. +15, h = lane >> 5), main chunk c of the row stored at
// c ^ swz_main(i), rope chunk c at c ^ swz_rope(i) (the bf16 tile layout).
__device__ __forceinline__ u32x8 q_raw_bf16(const lds_u8* smem, int qmain, int qrope, int lane, int n) {
  const int i = lane & 31, c0 = 4 * n + 2 * (lane >> 5);
  auto at = [&](int c) {
    return c < 64 ? qmain + i * kMainRow + ((c ^ swz_main(i)) << 4)
                  : qrope + i * kRopeRow + (((c - 64) ^ swz_rope(i)) << 4);
  };
  return cat8(lds_load<u32x4>(smem, at(c0)), lds_load<u32x4>(smem, at(c0 + 1)));
}
__device__ __forceinline__ bf16x8 fp8x8_to_bf16(uint32_t lo, uint32_t hi) {
  return cat(fp8x4_to_bf16(lo), fp8x4_to_bf16(hi));
}

// fp8 V^T fragment (kk, ct): one transposed 8-byte read (v_raw_f8), converted
// (v_frag_f8). The PV loop reads a fragment four products ahead and converts
// it two products ahead, so the conversion never waits on the read.
__device__ __forceinline__ u32x2 v_raw_f8(const lds_u8* smem, const LaneAddr& la, int vmain, int kk, int ct) {
  typedef int i32x2 __attribute__((ext_vector_type(2)));
  const i32x2 v = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
      (__attribute__((address_space(3))) i32x2*)(smem + vmain + 16 * kF8MainRow * kk + (la.va ^ (ct << 5))));
  return u32x2{(uint32_t)v[0], (uint32_t)v[1]};
}
__device__ __forceinline__ bf16x8 v_frag_f8(const lds_u8* smem, const LaneAddr& la, int vmain, int kk, int ct) {
  const u32x2 v = v_raw_f8(smem, la, vmain, kk, ct);
  return fp8x8_to_bf16(v[0], v[1]);
}

// V^T fragment for PV MFMAs (kk, ct): two transposed 8-byte reads. The XOR
// constants select the column tile (bits 6-7) and, for q = 1, flip
// c0 ^ g into c0 ^ (2 + g) (bit 5).
__device__ __forceinline__ bf16x8 v_frag(const lds_u8* smem, const LaneAddr& la, int vmain, int kk, int ct) {
  const int base = vmain + 16 * kMainRow * kk;
  const i16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4*)(smem + base + (la.va ^ (ct << 6))));
  const i16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4*)(smem + base + 8 * kMainRow + (la.va ^ ((ct << 6) | 32))));
  return cat(__builtin_bit_cast(bf16x4, v0), __builtin_bit_cast(bf16x4, v1));
}

__device__ __forceinline__ bf16x8 p_frag(const lds_u8* smem, const LaneAddr& la, int pbuf, int rb, int kk) {
  return lds_load<bf16x8>(smem, pbuf + (rb * 2 + kk) * 1024 + la.pl);
}

// Softmax of one tile on this wave's rows, in pieces that the pipelined step
// spreads over its MFMA slots. S^T register r of lane l is row l & 31, key
// key0 + 8 (r / 4) + r % 4 with key0 = tile start + 4 (l >> 5). A key is
// visible iff it is below the split's end and at most the row's position
// limit: lim = min(end - 1, pos_limit) - key0 (one compare per score). A
// row's reference max m_ref is its first visible tile's max (in base 2) and
// then stays fixed; a tile more than kRefSlack above it sets `over` (the item
// is recomputed with the row's true max, m_seen).
struct Softmax {
  float tmax, mu;
  bf16x8 pf[2];
  // fp8 PV: P 2^k of the lane's 16 keys as e4m3 (byte 4 g + e: key
  // 8 g + 4 h + e), 2^-k, and the E8M0 code 127 - k of 2^-k.
  u32x4 pf8;
  float lscale;
  int sbyte;
};
struct RowState {
  float m_ref, m_seen, l_part;
  float l_round;   // fp8 PV: the sum of the rounded weights (O's denominator)
  bool over;
};
// piece 0..3: scale and mask 4 scores, running max; piece 4: row max, the
// reference; pieces 5..12: two exponentials each. FAST (every score of the
// tile visible to every row of the wave, and a positive score scale) skips
// the mask and folds the scale into the exponent: the max of the raw scores
// times the scale is the max of the scaled scores, and exp2(s c - mu) is one
// fma.
// PV8 (P for the fp8 PV products): the exponentials come out as P 2^k, k a
// per-(row, tile) integer that puts the tile's largest P 2^k in (128, 256],
// inside e4m3's range (largest finite 448) with its full 4 significant bits;
// the PV product multiplies by the E8M0 scale 2^-k again, exactly, and the
// row sum adds the same rounded weights times 2^-k. Weights below 2^-17 of
// the tile's largest fall under e4m3's smallest subnormal and are dropped.
template <bool FAST, bool PV8 = false>
__device__ __forceinline__ void softmax_piece(int piece, Softmax& sm, f32x16& s, float score_c, int lim,
                                              RowState& rs) {
  if (piece < 4) {
    if constexpr (!FAST) {
      // The scores are scaled and masked in place (s is dead after this tile).
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 4 * piece + e;
        const float v = s[r] * score_c;
        s[r] = (8 * (r >> 2) + (r & 3) <= lim) ? v : -INFINITY;
      }
    }
    const float m4 = fmaxf(fmaxf(s[4 * piece], s[4 * piece + 1]), fmaxf(s[4 * piece + 2], s[4 * piece + 3]));
    sm.tmax = piece == 0 ? m4 : fmaxf(sm.tmax, m4);
  } else if (piece == 4) {
    const float tmax = FAST ? half_max(sm.tmax) * score_c : half_max(sm.tmax);
    rs.m_seen = fmaxf(rs.m_seen, tmax);
    // Until a row has seen a visible key its O and l are exactly zero, so its
    // reference may start at this tile's max without rescaling anything.
    if (rs.m_ref == -INFINITY) rs.m_ref = tmax;
    rs.over = rs.over || (tmax > rs.m_ref + kRefSlack);
    sm.mu = rs.m_ref == -INFINITY ? 0.0f : rs.m_ref;
    if constexpr (PV8) {
      // k = 8 - ceil(tmax - mu), kept in [-126, 126] (2^-k and 127 - k stay
      // normal floats and valid E8M0 codes; a tile past the clamp is either
      // entirely below 2^-118 of the reference or one that makes the item
      // run again). A row with no visible key in the tile takes k = 0.
      const float kf = tmax == -INFINITY ? 0.f : fminf(126.f, fmaxf(-126.f, 8.f - __builtin_ceilf(tmax - sm.mu)));
      const int k = (int)kf;
      sm.mu -= kf;
      sm.sbyte = 127 - k;
      sm.lscale = __int_as_float((127 - k) << 23);
    }
  } else if (piece < 13) {
    float pr2[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int r = 2 * (piece - 5) + e;
      // v_exp_f32 directly: arguments below -126 give 0 or a denormal, which
      // only drops weights under 2^-126 of the row's reference.
      const float pr = __builtin_amdgcn_exp2f(FAST ? __builtin_fmaf(s[r], score_c, -sm.mu) : s[r] - sm.mu);
      if constexpr (PV8) {
        pr2[e] = pr;
        rs.l_part = __builtin_fmaf(pr, sm.lscale, rs.l_part);
      } else {
        rs.l_part += pr;
        sm.pf[r >> 3][r & 7] = (__bf16)pr;
      }
    }
    if constexpr (PV8) {   // keys r, r + 1 (r = 2 (piece - 5)): half (piece - 5) & 1 of dword r / 4
      const int dw = (piece - 5) >> 1;
      if ((piece - 5) & 1) {
        sm.pf8[dw] = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(pr2[0], pr2[1], (int)sm.pf8[dw], true);
        // O is normalized by the sum of the rounded weights, so that it is a
        // weighted mean of V with exactly the weights the PV products use (a
        // dominant key's rounding then cancels between O's numerator and
        // denominator); the LSE keeps the exact sum.
        const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)sm.pf8[dw], false);
        const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)sm.pf8[dw], true);
        rs.l_round = __builtin_fmaf((lo[0] + lo[1]) + (hi[0] + hi[1]), sm.lscale, rs.l_round);
      } else {
        sm.pf8[dw] = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(pr2[0], pr2[1], (int)sm.pf8[dw], false);
      }
    }
  }
}
constexpr int kSoftmaxPieces = 13;

// ---------------------------------------------------------------------------
// In-kernel merge of one (row b, M tile m): rows m 128 .. m 128 + 127 of the
// row's block, n <= kMaxInKernelSplits bf16 partials each (consecutive
// partial slots from part0). Thread tid takes 32 (row, 8-column chunk) pairs.
__device__ __forceinline__ void merge_tile(const DecodeArgs& a, int m, int M, int n, int part0,
                                           int q0, int tid) {
  const int H = a.heads;
  const int64_t stride = (int64_t)a.q_len_max * H;   // between consecutive partial slots
  for (int i = 0; i < kRows * 64 / kDecodeThreads; ++i) {
    const int pair = tid + i * kDecodeThreads;
    const int rr = pair >> 6, c = pair & 63;
    const int r = m * kRows + rr;
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
        const bf16x8 src = *(const bf16x8*)(a.ws_o + (base + k * stride) * kDV + c * 8);
        const float wk = lk[k] * inv;   // an empty split's partial is 0 and its weight 0
        acc0 += wk * f32x4{(float)src[0], (float)src[1], (float)src[2], (float)src[3]};
        acc1 += wk * f32x4{(float)src[4], (float)src[5], (float)src[6], (float)src[7]};
      }
    }
    *(bf16x8*)dst = bf16x8{(__bf16)acc0[0], (__bf16)acc0[1], (__bf16)acc0[2], (__bf16)acc0[3],
                           (__bf16)acc1[0], (__bf16)acc1[1], (__bf16)acc1[2], (__bf16)acc1[3]};
    if (c == 0) a.lse[orow] = mx + __log2f(tot) * kLn2;
  }
}

// PV product p (0..31) of a tile: key half kk = p / 16, column tile
// ct = (p / 4) % 4, row block rb = p % 4. Each V^T fragment feeds four
// products and is read four products ahead; the key-half-1 P^T fragment of a
// row block replaces key half 0's after its last use.
template <bool KV_FP8>
__device__ __forceinline__ void pv_product(const lds_u8* smem, const LaneAddr& la, int vmain, int pbuf, int p,
                                           bf16x8 (&vb)[2], u32x2& vraw, bf16x8 (&pb)[kRowBlocks],
                                           f32x16 (&oacc)[kRowBlocks][kColTiles]) {
  const int kk = p >> 4, ct = (p >> 2) & 3, rb = p & 3;
  if (rb == 0 && p + 4 < 32) {
    if constexpr (KV_FP8) vraw = v_raw_f8(smem, la, vmain, (p + 4) >> 4, ((p + 4) >> 2) & 3);
    else vb[((p >> 2) + 1) & 1] = v_frag(smem, la, vmain, (p + 4) >> 4, ((p + 4) >> 2) & 3);
  }
  if constexpr (KV_FP8) {
    if (rb == 2 && p + 2 < 32) vb[((p >> 2) + 1) & 1] = fp8x8_to_bf16(vraw[0], vraw[1]);
  }
  oacc[rb][ct] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vb[(p >> 2) & 1], pb[rb], oacc[rb][ct], 0, 0, 0);
  if (kk == 0 && ct == 3) pb[rb] = p_frag(smem, la, pbuf, rb, 1);
}

// fp8 PV: one v_mfma_scale_f32_32x32x64_f8f6f4 covers 64 keys, the 32 of
// tile tA (even) and the 32 of tile tA + 1. The matrix core reads its 64 k
// positions as two blocks of 32, block b made of bytes 16 b .. 16 b + 15 of
// both lane halves and scaled by the E8M0 code of lane half b (checked
// against a host model of the instruction). So lane (row j, half h) of the
// B operand (P^T) holds its own 16 P^T values of tile tA in bytes 0..15 and
// those of tile tA + 1 in bytes 16..31 (byte 4 g + e: key 8 g + 4 h + e, the
// order of its S^T registers), and lane half b brings the scale of tile
// tA + b of row j; the A operand (V^T) takes the same keys with the same
// transposed reads as the bf16 PV products, from the two tiles. Every
// product's key positions match between A and B, and each block's P values
// share one scale, so O^T += V^T P^T exactly up to the fp8 rounding of P.
typedef int i32x8 __attribute__((ext_vector_type(8)));
__device__ __forceinline__ u32x8 v_frag8(const lds_u8* smem, const LaneAddr& la, int vA, int vB, int ct) {
  const u32x2 a0 = v_raw_f8(smem, la, vA, 0, ct), a1 = v_raw_f8(smem, la, vA, 1, ct);
  const u32x2 b0 = v_raw_f8(smem, la, vB, 0, ct), b1 = v_raw_f8(smem, la, vB, 1, ct);
  return u32x8{a0[0], a0[1], a1[0], a1[1], b0[0], b0[1], b1[0], b1[1]};
}
template <int RB>
__device__ __forceinline__ void mfma_pv8(f32x16& acc, const u32x8& v, const u32x8& p, uint32_t scale) {
  acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(__builtin_bit_cast(i32x8, v), __builtin_bit_cast(i32x8, p),
                                                       acc, 0, 0, 0, 0x7F7F7F7F, RB, (int)scale);
}

// Staged query operand j (link NQ - 2 kQLds + j) of this lane's row.
__device__ __forceinline__ int q_staged_off(const LaneAddr& la, int j) {
  return kOffQ8 + (la.w * 2 * kQLds + j) * 2048 + la.pl * 2;
}
__device__ __forceinline__ u32x8 q_staged(const lds_u8* smem, const LaneAddr& la, int j) {
  return cat8(lds_load<u32x4>(smem, q_staged_off(la, j)), lds_load<u32x4>(smem, q_staged_off(la, j) + 16));
}

// Publish P^T(t-1) of this wave's rows: bf16, or (PV8) fp8 at parity par
// with the row's scale code in byte w of its scale word (both lane halves
// of a row hold the same code and write the same byte).
template <bool PV8>
__device__ __forceinline__ void publish_p(lds_u8* smem, const LaneAddr& la, int pbuf, int par, int lane,
                                          const Softmax& sm) {
  if constexpr (PV8) {
    lds_store(smem, kOffP + par * kP8Bytes + la.w * 1024 + la.pl, sm.pf8);
    lds_store(smem, kOffP8Scale + par * 128 + (lane & 31) * 4 + la.w, (uint8_t)sm.sbyte);
  } else {
    lds_store(smem, pbuf + (la.w * 2 + 0) * 1024 + la.pl, sm.pf[0]);
    lds_store(smem, pbuf + (la.w * 2 + 1) * 1024 + la.pl, sm.pf[1]);
  }
}

// One pipeline step t, in two phases split by a barrier.
//   Phase A: QK(t) (if QK) from the K tile in (kmain, krope); the softmax
//     of tile t-1 (if PREV; scores in s_old, masked by lim_old)
//     runs between its products, one piece every kSmStride slots, and
//     publishes P^T(t-1) in pbuf. The matrix core works on QK(t) while the
//     VALU works on the softmax. The last QK product writes the scores of
//     tile t into s_old (the softmax has ended by then); the chain itself
//     accumulates in a variable local to the step.
//   Barrier (the step's only one): this wave first waits for its loads of
//     tile t+1; after it P^T(t-1) of every wave and tile t+1 are visible.
//   Phase B: PV(t-1) (if PREV) with V in vmain and P^T in pbuf; dma(i),
//     i < NDMA, issues later tiles' loads, one every kDmaStride products.
// A sched_barrier ends every slot, so the compiler keeps this order. K
// fragments are read kKDepth products ahead.
constexpr int kKDepth = 5;
constexpr int kSmStride = 2;
constexpr int kDmaStride = 3;
// QKM selects the QK products: 0 bf16 (36 k-steps, one per slot); 1 fp8 Q
// and KV (9 fp8 products, every fourth slot); 2 bf16 Q split in two fp8
// operands with fp8 KV (18 products, every second slot: hi then lo of each
// 64 dims). fp8 K is read kK8Depth products ahead; the softmax pieces keep
// their slots.
// PV8 (fp8 PV, fp8 KV): the softmax publishes P^T(t-1) in fp8 at parity
// par = (t-1) & 1 of the fp8 P^T buffers, and phase B multiplies only when
// pv_now: tiles tA = vmain and tA + 1 = vmain2 once both have their P^T, or
// tile tA alone (single: the item's last tile has an even index), whose
// second half of each product then gets zero P^T and scale 1.
template <bool QK, bool PREV, int NDMA, bool KV_FP8, bool FAST, int QKM, bool PV8 = false, typename QF, int NQ,
          typename Dma>
__device__ __forceinline__ void pipeline_step(lds_u8* smem, const LaneAddr& la, const QF (&qf)[NQ],
                                              int kmain, int krope, f32x16& s_old, float score_c,
                                              int lim_old, RowState& rs, int pbuf, int vmain,
                                              f32x16 (&oacc)[kRowBlocks][kColTiles], Dma&& dma,
                                              int vmain2 = 0, int par = 0, bool pv_now = false,
                                              bool single = false, int lane = 0, int rpar = 0) {
  static_assert(kSmStride * kSoftmaxPieces <= kKSteps, "softmax pieces fit between the QK products");
  static_assert(NDMA == 0 || kDmaStride * (NDMA - 1) < 32, "loads fit between the PV products");
  // bf16 K: fragments read kKDepth products ahead; fp8 K: kK8Depth.
  constexpr int kK8Depth = 3;
  constexpr bool QF8 = QKM != 0;
  static_assert(QKM == 0 ? (!KV_FP8 && NQ == kKSteps) : (KV_FP8 && NQ == QKM * kKSteps8),
                "Q fragments of the QK mode");
  bf16x8 kb[kKDepth];
  u32x8 k8[kK8Depth];
  constexpr bool kQStaged = PV8 && QKM == 2;
  u32x8 qr[3];
  Softmax sm;
  f32x16 s_cur;
  if constexpr (QK) {
    if constexpr (QF8) {
#pragma unroll
      for (int d = 0; d < kK8Depth; ++d) k8[d] = k_prod_f8(smem, la, kmain, krope, d);
    } else {
#pragma unroll
      for (int d = 0; d < kKDepth; ++d) kb[d] = k_frag(smem, la, kmain, krope, d);
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  constexpr int kSlotsA = QK ? kKSteps : kSoftmaxPieces * kSmStride;
#pragma unroll
  for (int s = 0; s < kSlotsA; ++s) {
    if constexpr (QK && QF8) {
      constexpr int kStride = 4 / QKM;   // slots per link
      if (s % kStride == 0) {
        const int n = s / kStride, p = n / QKM;   // link n of NQ, on K product p
        const u32x8 a = k8[p % kK8Depth];
        if (n % QKM == QKM - 1 && p + kK8Depth < kKSteps8)
          k8[p % kK8Depth] = k_prod_f8(smem, la, kmain, krope, p + kK8Depth);
        // The staged query operands (links NQ - 2 kQLds ..), read two links ahead.
        constexpr int kL0 = NQ - 2 * kQLds;
        if constexpr (kQStaged) {
          if (n + 2 >= kL0 && n + 2 < NQ) qr[(n + 2) % 3] = q_staged(smem, la, n + 2 - kL0);
        }
        const u32x8 b = (kQStaged && n >= kL0) ? qr[n % 3] : qf[n];
        if (n == 0) mfma8_qk_first(s_cur, a, b);
        else if (n + 1 < NQ) mfma8_qk(s_cur, a, b);
        else mfma8_qk_last(s_old, s_cur, a, b);   // s_old is dead: the softmax ended
      }
    } else if constexpr (QK) {
      const bf16x8 a = kb[s % kKDepth];
      if (s + kKDepth < kKSteps) kb[s % kKDepth] = k_frag(smem, la, kmain, krope, s + kKDepth);
      if (s == 0) mfma_qk_first(s_cur, a, qf[s]);
      else if (s + 1 < kKSteps) mfma_qk(s_cur, a, qf[s]);
      else mfma_qk_last(s_old, s_cur, a, qf[s]);   // s_old is dead: the softmax ended
    }
    if constexpr (PREV) {
      if (s % kSmStride == 0 && s / kSmStride < kSoftmaxPieces)
        softmax_piece<FAST, PV8>(s / kSmStride, sm, s_old, score_c, lim_old, rs);
      if (s == kSmStride * kSoftmaxPieces) publish_p<PV8>(smem, la, pbuf, par, lane, sm);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  if constexpr (PREV) {
    if constexpr (!QK) publish_p<PV8>(smem, la, pbuf, par, lane, sm);   // the slot loop ended with the last piece
  }
  // This wave's loads of tile t+1 (issued in step t-1, before this step's
  // slot-list load) have landed; after the barrier P^T(t-1) and tile t+1 are
  // visible to every wave. It is the step's only barrier.
  wait_vm<1>();
  __syncthreads();
  // Phase B.
  if constexpr (PV8) {
    if (PREV && pv_now) {   // uniform
      // Two halves of two row blocks each (P^T of two row blocks, 16
      // registers, at a time); the V^T fragments are read once per half.
      uint32_t sc = lds_load<uint32_t>(smem, kOffP8Scale + (rpar + (lane >> 5)) * 128 + (lane & 31) * 4);
      if (!QK && single) sc = lane >= 32 ? 0x7F7F7F7Fu : sc;   // tile tA + 1 does not exist
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        u32x8 pb8[2];
#pragma unroll
        for (int r = 0; r < 2; ++r) {
          pb8[r] = cat8(lds_load<u32x4>(smem, kOffP + rpar * kP8Bytes + (2 * hh + r) * 1024 + la.pl),
                        lds_load<u32x4>(smem, kOffP + (rpar + 1) * kP8Bytes + (2 * hh + r) * 1024 + la.pl));
          if (!QK && single) pb8[r][4] = pb8[r][5] = pb8[r][6] = pb8[r][7] = 0u;   // its half of each product is zero
        }
        u32x8 va[2];
        va[0] = v_frag8(smem, la, vmain, vmain2, 0);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int p = 0; p < 2 * kColTiles; ++p) {
          const int ct = p >> 1, r = p & 1, q = 8 * hh + p;
          if (r == 0 && ct + 1 < kColTiles) va[(ct + 1) & 1] = v_frag8(smem, la, vmain, vmain2, ct + 1);
          if (q % kDmaStride == 0 && q / kDmaStride < NDMA) dma(q / kDmaStride);
          if (hh == 0 && r == 0) mfma_pv8<0>(oacc[0][ct], va[ct & 1], pb8[0], sc);
          else if (hh == 0) mfma_pv8<1>(oacc[1][ct], va[ct & 1], pb8[1], sc);
          else if (r == 0) mfma_pv8<2>(oacc[2][ct], va[ct & 1], pb8[0], sc);
          else mfma_pv8<3>(oacc[3][ct], va[ct & 1], pb8[1], sc);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < NDMA; ++i) dma(i);
    }
    return;
  }
  bf16x8 pb[kRowBlocks];
  bf16x8 vb[2];
  u32x2 vraw;
  if constexpr (PREV) {
#pragma unroll
    for (int rb = 0; rb < kRowBlocks; ++rb) pb[rb] = p_frag(smem, la, pbuf, rb, 0);
    if constexpr (KV_FP8) vb[0] = v_frag_f8(smem, la, vmain, 0, 0);
    else vb[0] = v_frag(smem, la, vmain, 0, 0);
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int p = 0; p < 32; ++p) {
    if (p % kDmaStride == 0 && p / kDmaStride < NDMA) dma(p / kDmaStride);
    if constexpr (PREV) pv_product<KV_FP8>(smem, la, vmain, pbuf, p, vb, vraw, pb, oacc);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// MERGE: the variant for in-kernel-merge plans (the default variant carries
// none of that code, which would cost the hot loops registers).
// PV8: the fp8 PV products (fp8 KV only).
template <bool Q_FP8, bool KV_FP8, bool MERGE, bool PV8>
__global__ __launch_bounds__(kDecodeThreads, 1) void decode_kernel(DecodeArgs a) {
  static_assert(KV_FP8 || !PV8, "fp8 PV needs fp8 KV");
  __shared__ __attribute__((aligned(16))) unsigned char smem_raw[kSmemBytes];
  lds_u8* smem = (lds_u8*)smem_raw;
  using LY = Layout<KV_FP8, PV8>;
  using Dma = TileDma<KV_FP8>;
  constexpr int QKM = !KV_FP8 ? 0 : Q_FP8 ? 1 : 2;   // QK products: bf16, fp8, split bf16 Q

  const int tid = threadIdx.x;
  const int w_k = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int H = a.heads;
  const unsigned char* kv = (const unsigned char*)a.kv;
  const float q_scale = a.q_scale ? *a.q_scale : 1.0f;
  const float kv_scale = a.kv_scale ? *a.kv_scale : 1.0f;
  // (wave-uniform: kept in a scalar register, never spilled to scratch)
  const float score_c = __builtin_bit_cast(
      float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, a.score_scale_log2 * q_scale * kv_scale)));

  const int g = blockIdx.x;
  const int it0 = ldc(a.plan, a.off_work_indptr + g), it1 = ldc(a.plan, a.off_work_indptr + g + 1);
  for (int it = it0; it < it1; ++it) {
    // An opaque copy of the wave index: the LDS offsets and addresses derived
    // from it are computed in the item instead of being hoisted out of the
    // item loop into scalar registers, which the compiler then spilled.
    const int w = opaque_s(w_k);
    const int s = ldc(a.plan, a.off_item_split + it);
    const int m = ldc(a.plan, a.off_item_m + it);
    const int b = ldc(a.plan, a.off_split_row + s);
    const int part = ldc(a.plan, a.off_split_part + s);
    const int q0 = ldc(a.qo_indptr, b), q_b = ldc(a.qo_indptr, b + 1) - q0;
    const int kv0 = ldc(a.kv_indptr, b), L = ldc(a.kv_indptr, b + 1) - kv0;
    const int s0 = ldc(a.plan, a.off_split_indptr + b);
    const int nsplit = ldc(a.plan, a.off_split_indptr + b + 1) - s0;
    int begin, end;
    if (a.uniform_ranges) {   // split k of n covers [k L / n, (k + 1) L / n) of the live length
      begin = (int)((int64_t)(s - s0) * L / nsplit);
      end = (int)((int64_t)(s - s0 + 1) * L / nsplit);
    } else {
      begin = ldc(a.plan, a.off_split_begin + s);
      end = ldc(a.plan, a.off_split_end + s);
    }
    const int M = q_b * H;
    if (m * kRows >= M) continue;   // no query row in this tile (ragged block); uniform
    const int ntiles = (end - begin + kNT - 1) / kNT;

    // ---- this wave's query rows: m 128 + 32 w + (lane & 31)
    // Lane-derived values are recomputed from a lane id computed afresh
    // (lane_now): kept live across the item loop they would be spilled, and
    // each reload from scratch is a vector-memory access whose wait also waits
    // for every earlier load and store (the previous item's O stores, the
    // tile loads in flight).
    const int ilane = lane_now();
    const int mr = m * kRows + 32 * w + (ilane & 31);
    const bool row_ok = mr < M;
    // (rows past the block's end get a token index past q_b; nothing of
    // theirs is written)
    const int tok = div_small(mr, opaque_s(H));
    // Causal mask on global positions: local key j sits at j * world + rank
    // of the row's P keys over all shards, token tok at P - q_b + tok; the
    // visible local keys are j <= (P - q_b + tok - rank) / world (one shard:
    // j <= L - q_b + tok). Rows past the end of the block are computed but
    // never written; they take the non-causal limit.
    const int Pk = a.kv_len_global ? ldc(a.kv_len_global, b) : L;
    const int qpos = Pk - q_b + tok - a.dcp_rank;
    const int causal_lim = qpos < 0 ? -1 : a.dcp_world == 1 ? qpos : qpos / opaque_s(a.dcp_world);
    const int pos_limit = (a.causal && row_ok) ? causal_lim : (L - 1);
    const int key_last = min(end - 1, pos_limit);   // last visible key of this row in the split
    // The B operand of S^T = K Q^T. bf16 KV: lane holds, for k-step ks, the
    // 8 dims that the K fragment's lane half h = lane >> 5 holds,
    // 16 ks + 8 h .. +7, i.e. 8-element unit 2 ks + h.
    // With fp8 Q and KV the raw fp8 bytes of product p: 16-byte units
    // 4 p + h and 4 p + 2 + h. With bf16 Q and fp8 KV the same 32 elements
    // (bf16 units 8 p + 2 h, +1, 8 p + 4 + 2 h, +1) split into hi (qf[2 p])
    // and lo (qf[2 p + 1]); score_row then carries the row's 2^-A.
    std::conditional_t<(QKM > 0), u32x8, bf16x8> qf[QKM == 0 ? kKSteps : QKM * kKSteps8];
    float score_row = score_c;
    // Query row (tok, head) of the block is row mr of the request row's
    // [q_b * H, 576] block. Rows past the block's end (computed, never
    // written) take a copy of its last row; the split of bf16 queries for
    // fp8 KV sets them to zero instead.
    constexpr int kQElem = Q_FP8 ? 1 : 2;
    const unsigned char* qblock = (const unsigned char*)a.q + (int64_t)q0 * H * (kDLat * kQElem);
    // Every mode but fp8 queries with bf16 KV stages its rows through LDS
    // (in the tile layout of the query dtype). The first slot lists of pass 0
    // go out first, so that their latency overlaps the staging.
    constexpr bool kStageQ = !(Q_FP8 && !KV_FP8);
    // fp8 queries and KV without fp8 PV: staged above the tile ring, so pass
    // 0's first tiles are issued before the queries are waited for.
    constexpr bool kQAbove = QKM == 1 && !PV8;
    using QS = std::conditional_t<kQAbove, QStageAbove, QStage<Q_FP8>>;
    if constexpr (kStageQ) {
      if (ntiles > 0) {
#pragma unroll
        for (int t = 0; t < 4; ++t) issue_slots(a.kv_indices, kv0, begin, end, t, smem, w, ilane);
#pragma unroll
        for (int q = 0; q < kWaves; ++q)
          TileDma<Q_FP8>::all(qblock, m * kRows + 32 * q + (ilane & 31), (uint32_t)(M - 1), smem,
                              QS::main(q), QS::rope(q), w, ilane);
        if constexpr (kQAbove) {
          // This wave's slot lists of tiles 0 and 1 have landed (two slot
          // lists and the query loads may still be in flight); then the
          // pass prologue's loads of tiles 0 and 1, in its order, and the
          // queries land (those loads may still be in flight).
          wait_vm<2 + kWaves * TileDma<Q_FP8>::n>();
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            const int plane = lane_now();
            issue_slots(a.kv_indices, kv0, begin, end, t + 2, smem, w, plane);
            if (t < ntiles)
              Dma::all(kv, read_slots(smem, t, w, plane), a.max_slot, smem, LY::main(t), LY::rope(t), w, plane);
          }
          if (ntiles > 1) wait_vm<2 * (1 + Dma::n)>();
          else wait_vm<2 + Dma::n>();
        } else {
          wait_vm<0>();
        }
        __syncthreads();   // every wave's query rows and slot lists have landed
        const int ql = lane_now();
        if constexpr (QKM == 0) {
          const LaneAddr la_q = lane_addr<false>(ql, w);
#pragma unroll
          for (int ks = 0; ks < kKSteps; ++ks) qf[ks] = k_frag(smem, la_q, QS::main(w), QS::rope(w), ks);
        } else if constexpr (QKM == 1) {
          const LaneAddr la_q = lane_addr<true>(ql, w);
#pragma unroll
          for (int p = 0; p < kKSteps8; ++p) qf[p] = k_prod_f8(smem, la_q, QS::main(w), QS::rope(w), p);
        } else {   // raw bf16 here; split once the item's first loads are out
          const bool keep = m * kRows + 32 * w + (ql & 31) < M;
#pragma unroll
          for (int n = 0; n < 2 * kKSteps8; ++n) {
            const u32x8 v = q_raw_bf16(smem, QS::main(w), QS::rope(w), ql, n);
            qf[n] = keep ? v : u32x8{};
          }
        }
        // the tile loads below rewrite the staging region (above the tile
        // ring it is next written by the P^T of step 1, after step 0's barrier)
        if constexpr (!kQAbove) __syncthreads();
      }
    } else {
      // (opaque: computed here rather than hoisted and spilled)
      const unsigned char* qsrc = qblock + (uint32_t)opaque(min(mr, M - 1)) * (uint32_t)(kDLat * kQElem);
      const int h = ilane >> 5;
      const u32x2* src = (const u32x2*)qsrc;
#pragma unroll
      for (int ks = 0; ks < kKSteps; ++ks) {
        const u32x2 v = src[2 * ks + h];
        qf[ks] = cat(fp8x4_to_bf16(v[0]), fp8x4_to_bf16(v[1]));
      }
    }

    // Pass 0 fixes each row's reference at its first visible tile's max. In
    // the rare case that a later tile exceeds it by more than kRefSlack, the
    // item runs once more with every row's reference at its true max.
    RowState rs{-INFINITY, -INFINITY, 0.f, 0.f, false};
    f32x16 oacc[kRowBlocks][kColTiles];
    for (int pass = 0; pass < 2; ++pass) {
      rs.l_part = 0.f;
      rs.l_round = 0.f;
      rs.over = false;
#pragma unroll
      for (int rb = 0; rb < kRowBlocks; ++rb)
#pragma unroll
        for (int ct = 0; ct < kColTiles; ++ct) oacc[rb][ct] = f32x16{};
      if (ntiles > 0) {
        // Prologue: slot lists of tiles 0..3 (pass 0 of a staged item has
        // them already), then the loads of tiles 0 and 1, each preceded by
        // one slot-list load so that every later wait count has the same
        // form; tile 0 lands.
        // The lane-derived addresses here are computed where they are used
        // (from a fresh lane id): shared with the item head's they would be
        // kept live across the query staging and spilled, and a reload's wait
        // would also wait for the tile loads issued before it.
        if (!kStageQ || pass > 0) {
#pragma unroll
          for (int t = 0; t < 4; ++t) issue_slots(a.kv_indices, kv0, begin, end, t, smem, w, lane_now());
          wait_vm<0>();
        }
        if (!kQAbove || pass > 0) {   // (pass 0 above the ring: issued with the queries)
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            const int plane = lane_now();
            issue_slots(a.kv_indices, kv0, begin, end, t + 2, smem, w, plane);
            if (t < ntiles)
              Dma::all(kv, read_slots(smem, t, w, plane), a.max_slot, smem, LY::main(t), LY::rope(t), w, plane);
          }
        }
        if constexpr (QKM == 2) {
          if (pass == 0) {
            score_row = score_c * split_q_rows(qf);
            if constexpr (PV8) {   // the last products' operands wait in LDS (read back by this lane only)
              const LaneAddr la_q = lane_addr<KV_FP8>(ilane, w);
#pragma unroll
              for (int j = 0; j < 2 * kQLds; ++j) {
                const u32x8 v = qf[2 * (kKSteps8 - kQLds) + j];
                lds_store(smem, q_staged_off(la_q, j), u32x4{v[0], v[1], v[2], v[3]});
                lds_store(smem, q_staged_off(la_q, j) + 16, u32x4{v[4], v[5], v[6], v[7]});
              }
            }
          }
        }
        if (ntiles > 1) wait_vm<1 + Dma::n>();
        else wait_vm<1>();
        __syncthreads();

        // s_old: the previous tile's scores, consumed by its softmax in the
        // next step.
        f32x16 s_old;
        // Step t: QK(t) if t < ntiles, the softmax of tile t-1 and PV(t-1) if
        // t >= 1; tile t+2's loads are issued in phase B, after the step's
        // barrier (which also publishes tile t+1). QK, PREV and DMA are
        // template flags, so the hot loop carries no per-slot branch; FAST
        // selects the unmasked softmax for tile t-1.
        auto run_step = [&](int t, auto QKc, auto PREVc, auto DMAc, auto FASTc) {
          constexpr bool DO_QK = decltype(QKc)::value, PREV = decltype(PREVc)::value;
          constexpr bool DO_DMA = decltype(DMAc)::value, FAST = decltype(FASTc)::value;
          const int dlane = lane_now();
          // (opaque: no per-loop copies of this base derived up front and
          // spilled. An opaque copy is an assembly statement, which memory
          // accesses are not moved across: it comes before the slot-list
          // read below, which the scheduler then interleaves with the first
          // K-fragment reads.)
          const int lim_old = opaque(key_last) - (begin + (t - 1) * kNT + 4 * (dlane >> 5));
          issue_slots(a.kv_indices, kv0, begin, end, t + 4, smem, w, dlane);
          const TileSrc<KV_FP8> src = Dma::src(kv, DO_DMA ? read_slots(smem, t + 2, w, dlane) : 0, a.max_slot, w, dlane);
          const int dm = LY::main(t + 2), dr = LY::rope(t + 2);
          auto dma = [&](int i) {
            Dma::op(i, kv, src, lds_addr_of(smem), dm, dr, w, dlane);
          };
          const LaneAddr la_s = lane_addr<KV_FP8>(dlane, w);
          if constexpr (PV8) {
            // PV of tiles tA = (t - 1) & ~1 and tA + 1 once both have their
            // P^T (t even), or of tA alone in the last step when it is the
            // item's last tile.
            // (the step without QK is the last one, t = ntiles). Alone, tile
            // tA also stands in for the second tile's V^T: whatever another
            // buffer holds (an older tile, or LDS never written, possibly NaN
            // codes) must not meet the zero P^T, since 0 x NaN is NaN.
            const int tA = (t - 1) & ~1;
            const bool single = !DO_QK && (t & 1) != 0;
            pipeline_step<DO_QK, PREV, DO_DMA ? Dma::n : 0, KV_FP8, FAST, QKM, true>(
                smem, la_s, qf, LY::main(t), LY::rope(t), s_old, score_row, lim_old, rs, 0, LY::main(tA), oacc,
                dma, LY::main(single ? tA : tA + 1), (t - 1) & 3, !DO_QK || (t & 1) == 0, single, dlane, tA & 3);
          } else {
            pipeline_step<DO_QK, PREV, DO_DMA ? Dma::n : 0, KV_FP8, FAST, QKM>(
                smem, la_s, qf, LY::main(t), LY::rope(t), s_old, score_row, lim_old, rs, p_buf(t + 1),
                LY::main(t + 11), oacc, dma);
          }
        };
        using T_ = std::true_type;
        using F_ = std::false_type;
        // ntiles + 1 steps: 0 .. ntiles
        if (ntiles > 2) run_step(0, T_{}, F_{}, T_{}, F_{});
        else run_step(0, T_{}, F_{}, F_{}, F_{});
        // The steady-state steps take the unmasked softmax while every key of
        // the tile is visible to every row of this wave: tile t is, iff
        // lim >= 27 on every lane (a lane's keys sit at most 27 past its
        // key0), i.e. for t < nfast, a prefix of the tiles (uniform).
        const int slack = __builtin_amdgcn_readfirstlane(
            wave_min_i32(key_last - begin - 4 * (ilane >> 5) - 27));
        const int nfast = score_c > 0.f && slack >= 0 ? slack / kNT + 1 : 0;
        int t = 1;
        for (; t + 2 < ntiles && t - 1 < nfast; ++t) run_step(t, T_{}, T_{}, T_{}, T_{});
        for (; t + 2 < ntiles; ++t) run_step(t, T_{}, T_{}, T_{}, F_{});
        for (t = ntiles > 3 ? ntiles - 2 : 1; t < ntiles; ++t) run_step(t, T_{}, T_{}, F_{}, F_{});
        run_step(ntiles, F_{}, T_{}, F_{}, F_{});
        wait_vm<0>();
      }
      // Did any row of the item overflow its reference? (uniform) One
      // barrier publishes the waves' flags and the rows' O denominators for
      // the epilogue; a pass 1 rewrites both before they are read again.
      if (lane_now() == 0) lds_store(smem, kOffMisc + 4 * w, (uint32_t)(__ballot(rs.over) != 0));
      {
        // (cross-lane sums run on every lane, outside the lane < 32 branch)
        const float l_o = half_sum(PV8 ? rs.l_round : rs.l_part);   // O's denominator
        const int el = lane_now();
        if (el < 32) lds_store(smem, kOffL + (w * 32 + el) * 4, l_o);
      }
      __syncthreads();
      const u32x4 ov = lds_load<u32x4>(smem, kOffMisc);
      if (pass == 1 || (ov[0] | ov[1] | ov[2] | ov[3]) == 0u) {
        // O normalized and staged here, in the block that produced the
        // accumulators: staged after the loop, they would be live across its
        // exit, where the register allocator reshuffled them and spilled a
        // dozen to scratch (each reload a wait of its own in the epilogue).
        // O leaves through LDS so that the stores are whole rows: the item's
        // query rows r = m 128 .. m 128 + 127 are consecutive rows of O (index
        // q0 H + r) and of its partial slot (index (part q_len_max) H + r).
        // All 128 rows are staged at once in bf16 (1 KB per row, 128 KB of
        // the tile region), 16-byte chunk c of row r at c ^ (r & 15).
        const int el = lane_now();
        const int hh = el >> 5;
        // (column tiles outer: the register allocator then permutes and
        // spills fewer of the accumulators here)
        float inv_rb[kRowBlocks];
#pragma unroll
        for (int rb = 0; rb < kRowBlocks; ++rb) {
          const float l = lds_load<float>(smem, kOffL + (32 * rb + (el & 31)) * 4);
          inv_rb[rb] = l > 0.f ? kv_scale / l : 0.f;
        }
#pragma unroll
        for (int ct = 0; ct < kColTiles; ++ct) {
#pragma unroll
          for (int rb = 0; rb < kRowBlocks; ++rb) {
            const int r = 32 * rb + (el & 31);
            const float inv = inv_rb[rb];
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) {
              const f32x16& v = oacc[rb][ct];
              // columns 4 c' .. 4 c' + 3 with c' = 32 w + 8 ct + 2 gq + hh: half hh
              // of 16-byte chunk 16 w + 4 ct + gq
              const int c = 16 * w + 4 * ct + gq;
              const bf16x4 x{(__bf16)(v[4 * gq] * inv), (__bf16)(v[4 * gq + 1] * inv),
                             (__bf16)(v[4 * gq + 2] * inv), (__bf16)(v[4 * gq + 3] * inv)};
              lds_store(smem, r * (kDV * 2) + ((c ^ (r & 15)) << 4) + 8 * hh, x);
            }
          }
        }
        break;
      }
      rs.m_ref = rs.m_seen;   // pass 1: no tile can exceed the true max
    }

    // Epilogue: the staged O written, then the LSE (stored last, so that no
    // wait inside the epilogue waits for its store).
    const float l_row = half_sum(rs.l_part);
    const float lse = l_row > 0.f ? (rs.m_ref + __log2f(l_row)) * kLn2 : -INFINITY;
    {
      // (a fresh lane id: the addresses below are computed here rather than
      // hoisted out of the item loop and kept live across it)
      const int el = lane_now();
      const int64_t orow0 = part < 0 ? (int64_t)q0 * H + (int64_t)m * kRows
                                     : (int64_t)part * a.q_len_max * H + (int64_t)m * kRows;
      __syncthreads();
      const int nrows = min(kRows, M - m * kRows);   // rows of the item inside the block
      uint16_t* const dst0 = part < 0 ? a.o : a.ws_o;   // bf16 O, or the split's partial O
      // A lane takes one staged chunk (8 columns) of a row per store: row
      // r = 4 i + w (uniform), chunk el. The chunks of a batch are all read
      // before its stores, so the LDS latency is paid once per batch (two
      // batches of 16: the queries are dead here, so the registers are free;
      // one batch of 32 made the compiler spill inside the step loops).
      constexpr int kStores = kRows / kWaves, kBatch = 16;
#pragma unroll
      for (int i0 = 0; i0 < kStores; i0 += kBatch) {
        bf16x8 v[kBatch];
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
          const int r = kWaves * (i0 + j) + w;
          v[j] = lds_load<bf16x8>(smem, r * (kDV * 2) + ((el ^ (r & 15)) << 4));
        }
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
          const int r = kWaves * (i0 + j) + w;
          if (r < nrows) *(bf16x8*)(dst0 + (orow0 + r) * kDV + 8 * el) = v[j];
        }
      }
      // The LSE of this wave's rows: row mr of the block is (token tok, head),
      // index (q0 + tok) H + head = q0 H + mr.
      const int mr_e = m * kRows + 32 * w + (el & 31);
      if (el < 32 && mr_e < M) {
        if (part < 0) a.lse[(int64_t)q0 * H + mr_e] = lse;
        else a.ws_lse[(int64_t)part * a.q_len_max * H + mr_e] = lse;
      }
      __syncthreads();
    }

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
        merge_tile(a, m, M, nsplit, ldc(a.plan, a.off_split_part + s0), q0, tid);
        if (tid == 0) a.counters[b * a.u + m] = 0;
      }
      __syncthreads();
    }
  }
}

// ---------------------------------------------------------------------------
// Gather test hook: one block per split; every tile goes through the decode
// kernel's loader into tile 0, then is copied out of LDS with the swizzle
// undone (fp8 converted exactly to bf16, as the decode does in registers).
template <bool KV_FP8>
__global__ __launch_bounds__(kDecodeThreads) void gather_kernel(GatherArgs a) {
  __shared__ __attribute__((aligned(16))) unsigned char smem_raw[kTilesEnd];
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
    TileDma<KV_FP8>::all(kv, slot, a.max_slot, smem, dma_main<KV_FP8>(0), dma_rope<KV_FP8>(0), wave, lane);
    wait_vm_all();
    __syncthreads();
    for (int p = tid; p < kNT * 72; p += kDecodeThreads) {
      const int row = p / 72, chunk = p - row * 72;   // chunk: 8 latent dims
      if (key0 + row < end) {
        u32x4 v;
        if constexpr (!KV_FP8) {
          const int off = chunk < 64 ? LY::main(0) + row * kMainRow + ((chunk ^ swz_main(row)) << 4)
                                     : LY::rope(0) + row * kRopeRow + (((chunk - 64) ^ swz_rope(row)) << 4);
          v = lds_load<u32x4>(smem, off);
        } else {   // 8 fp8 bytes, half of a 16-byte chunk, converted exactly
          const int c = chunk < 64 ? chunk : chunk - 64;
          const int off = chunk < 64
                              ? LY::main(0) + row * kF8MainRow + (((c >> 1) ^ swz_f8(row)) << 4) + 8 * (c & 1)
                              : LY::rope(0) + (row >> 3) * 1024 + (row & 7) * kF8RopeRow +
                                    (((c >> 1) ^ swz_f8_rope(row)) << 4) + 8 * (c & 1);
          const u32x2 x = lds_load<u32x2>(smem, off);
          v = __builtin_bit_cast(u32x4, cat(fp8x4_to_bf16(x[0]), fp8x4_to_bf16(x[1])));
        }
        *(u32x4*)(a.dense + (dense0 + key0 + row) * kDLat + chunk * 8) = v;
      }
    }
    __syncthreads();
  }
}

}  // namespace

// (fp8 PV plans never merge inside the decode kernel: the planner refuses
// that combination.)
template <bool MERGE>
const void* decode_fn(bool q_fp8, bool kv_fp8, bool pv_fp8) {
  if (kv_fp8 && pv_fp8) {
    if constexpr (MERGE) return nullptr;
    else return q_fp8 ? (const void*)decode_kernel<true, true, false, true> : (const void*)decode_kernel<false, true, false, true>;
  }
  if (!q_fp8 && !kv_fp8) return (const void*)decode_kernel<false, false, MERGE, false>;
  if (!q_fp8 && kv_fp8) return (const void*)decode_kernel<false, true, MERGE, false>;
  if (q_fp8 && !kv_fp8) return (const void*)decode_kernel<true, false, MERGE, false>;
  return (const void*)decode_kernel<true, true, MERGE, false>;
}

hipError_t launch_decode(const DecodeArgs& a, bool q_fp8, bool kv_fp8, bool pv_fp8, int grid, hipStream_t st) {
  void* args[] = {(void*)&a};
  const void* fn = a.inkernel_max_splits > 1 ? decode_fn<true>(q_fp8, kv_fp8, pv_fp8)
                                             : decode_fn<false>(q_fp8, kv_fp8, pv_fp8);
  if (!fn) return hipErrorInvalidValue;
  return hipLaunchKernel(fn, dim3(grid), dim3(kDecodeThreads), args, 0, st);
}

hipError_t launch_gather(const GatherArgs& a, bool kv_fp8, int splits, hipStream_t st) {
  void* args[] = {(void*)&a};
  const void* fn = kv_fp8 ? (const void*)gather_kernel<true> : (const void*)gather_kernel<false>;
  return hipLaunchKernel(fn, dim3(splits), dim3(kDecodeThreads), args, 0, st);
}

}  // namespace mla
