// splitkv_partial_mfma.hip -- partial kernel of split-KV grouped-query decode
// attention for gfx950 (CDNA4), matrix-core form, used for head_dim 64, 128
// and 256.
//
// Same contract as the vector-ALU kernel: one workgroup (4 waves; 8 at
// head_dim 256) per (split, KV head, sequence) on a static grid
// dim3(n_splits, n_kv_head, batch), the live length read from positions[] on
// the device ("10 · R4 — decode
// split-attention dim-parallel rewrite", section 2.2), all G query heads of
// the KV head served by one read of each K/V row ("Red Lite dev35 —
// long-context decode: grouped split-K attention", Change), online softmax per
// head and one (mx, S, oc) record per query head ("10 · R4", section 2.1).
//
// Why matrix cores: grouping turns the scores of a row tile into a real dense
// contraction, S[rows][heads] = K[rows][hd] · Q[heads][hd]ᵀ, and the output
// update into O[hd][heads] += Vᵀ[hd][rows] · P[rows][heads]. Done with
// vector FMAs these cost 2*G*hd FMAs per row plus the dot-product
// reductions, which measured at about 78 wave instructions per KV row for
// 28q/4kv hd128 (the VALU issue limit lands near half of the HBM rate). On
// the matrix cores they take one v_mfma_f32_16x16x32_f16 per 16 rows and 32
// dims (scores, accumulated in two chains of even and odd 32-dim steps) and
// one v_mfma_f32_16x16x16_f16 per 16 rows and 16 dims (output).
//
// Precision: the MFMA takes fp16 operands and accumulates in fp32. K and V
// are fp16 already. q (scaled by scale*log2(e)) and the softmax weights p are
// fp32; each is split into fp16 hi = fp16(x) and lo = fp16(x - hi), which
// carry about 22 significant bits together. The 16 MFMA columns hold the G
// heads' hi parts in columns 0..7 and their lo parts in columns 8..15, so one
// MFMA computes both halves and a DPP row rotation by 8 adds them. (Several
// query rows of one sequence can share the columns as (row, head) pairs; up
// to 16 pairs use two column blocks, hi parts in one and lo parts in the
// other, each product run once per block.)
//
// Start of a workgroup: the live length is read first and wave 0 issues the
// query loads while it is in flight (they do not depend on it), every wave
// then issues its first tile's loads, wave 0 converts the queries into the
// MFMA operand once and the waves read it from LDS after one barrier. End:
// the waves' states are merged through LDS into one record per query head; a
// split of at most one tile has rows only in wave 0, which writes the records
// itself.
//
// Data flow of one wave over a tile of 16 rows (a workgroup's waves take
// interleaved tiles):
//   loads: K and V with 16-byte loads that each cover whole 2*hd-byte rows
//      (one instruction = 64 lanes = 4 rows at hd 128), so every cache line
//      an instruction touches is used in full. (A K load shaped like the
//      MFMA operand, 16 rows x 64 bytes per instruction, measured ~1.2 us
//      slower per 64 MB launch.)
//   staging: the tile's K and V rows go from the load registers into the
//      wave's LDS slice; the next tile's loads are issued into the same
//      registers once the staged tile is computed (one tile per wave in
//      flight at most: fewer bytes queued in the memory system measured
//      faster than keeping every wave's next tile in flight). At head_dim 256
//      the next tile's K (V) loads leave as soon as the current K (V) is
//      staged.
//   K: LDS rows 16 bytes past a multiple of 256 bytes apart, so the 16 rows
//      of an operand read fall in 16 different bank groups; read back as the
//      A operand of S = K·Q'ᵀ: lane l holds row l % 16, dims 32*ks + 8*(l/16);
//   scores: D lane l holds rows 4*(l/16)+r of its column l % 16 -> max over
//      the tile by in-lane max and two cross-group exchanges,
//      p = exp2(s - m);
//   p: already in the B-operand layout of O += Vᵀ·P (4 rows per lane);
//   V: LDS rows padded by 32 bytes against bank conflicts, read back with
//      the gfx950 transposing LDS read (ds_read_b64_tr_b16), which delivers
//      four rows of one dim per lane: the A operand of Vᵀ·P on
//      v_mfma_f32_16x16x16_f16.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "splitkv_internal.h"
#include "splitkv_partial_common.h"

namespace splitkv {
namespace {

using detail::dpp_mov;
using detail::fast_exp2;
using detail::neg_inf;

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef short short4v __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) short4v lds_short4v;

constexpr int kRor8 = 0x128;  // DPP row_ror:8 (rotate by 8 within 16 lanes)
constexpr float kLazyLog2 = 8.0f;  // reference-max lag allowed (base-2 units)

constexpr int kTileRows = 16;

template <int HD>
struct MGeo {
  static constexpr int KS = HD / 32;               // q·k k-steps of 32 dims
  static constexpr int DB = HD / 16;               // p·v output blocks of 16 dims
  static constexpr int LPR = HD / 8;               // lanes per row in a load
  static constexpr int RPI = 64 / LPR;             // rows per load instruction
  static constexpr int NL = kTileRows / RPI;       // loads per tile and tensor
  static constexpr int KSTR = HD * 2 + 16;         // LDS bytes per staged K row
  static constexpr int VSTR = HD * 2 + 32;         // LDS bytes per staged V row
  static constexpr int KTILE = kTileRows * KSTR;   // staged K bytes
  // LDS bytes per wave: staged K and V; after the last tile the same bytes
  // hold the wave's unnormalised output for the workgroup merge.
  static constexpr int SLICE = KTILE + kTileRows * VSTR;
  static_assert(HD % 32 == 0 && HD <= 256, "head_dim");
};

// Waves per workgroup: 4 (one per SIMD), 8 at head_dim 256. A head_dim-256
// tile is computed for longer and a split holds few tiles (8,400 rows over 96
// to 128 splits: 5-6 tiles), so with 4 waves some waves take a second tile
// after their first; 8 waves put every tile of a split of up to 128 rows in
// the first round (16q/2kv at 8,400 rows: 7.23 against 7.39 us at 96 splits,
// 7.60 against 7.84 at 128). The 8-wave workgroup uses 143 KB of LDS, so one
// fits a compute unit.
template <int HD>
struct MWaves {
  static constexpr int W = HD >= 256 ? 8 : 4;
  static constexpr int kThr = 64 * W;
};

// One tile's K and V rows as loaded: load i holds rows RPI*i + lane / LPR,
// dims 8*(lane % LPR) .. +7.
template <int HD>
struct TileRegs {
  uint4 k[MGeo<HD>::NL];
  uint4 v[MGeo<HD>::NL];
};

__device__ __forceinline__ half8 as_half8(const uint4 &u) {
  return __builtin_bit_cast(half8, u);
}

// Order this wave's LDS accesses: a compiler barrier around the wave's own
// in-order LDS traffic (the staged tile is private to the wave).
__device__ __forceinline__ void wave_lds_fence() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// x + (x of the lane 8 places along, within each row of 16): the hi + lo
// column sum. All lanes are valid sources for a rotation, so the move is
// written with bound_ctrl set, which lets the compiler fold it into the add
// as a DPP operand.
__device__ __forceinline__ float add_ror8(float x) {
  return x + __builtin_bit_cast(
                 float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x),
                                                    kRor8, 0xF, 0xF, true));
}

// Reductions across the four 16-lane rows of a wave (the 4 row groups of an
// MFMA column). v_permlane16_swap / v_permlane32_swap given (x, x) return, in
// every lane, the pair (x of the partner lane with that bit clear, x of the
// one with it set): a VALU exchange instead of an LDS permute round trip, and
// both lanes of a pair combine the two values in the same order.
__device__ __forceinline__ float pair16_max(float x) {
  const int b = __builtin_bit_cast(int, x);
  const auto r = __builtin_amdgcn_permlane16_swap(b, b, false, false);
  return fmaxf(__builtin_bit_cast(float, (int)r[0]),
               __builtin_bit_cast(float, (int)r[1]));
}
__device__ __forceinline__ float pair32_max(float x) {
  const int b = __builtin_bit_cast(int, x);
  const auto r = __builtin_amdgcn_permlane32_swap(b, b, false, false);
  return fmaxf(__builtin_bit_cast(float, (int)r[0]),
               __builtin_bit_cast(float, (int)r[1]));
}
__device__ __forceinline__ float pair16_sum(float x) {
  const int b = __builtin_bit_cast(int, x);
  const auto r = __builtin_amdgcn_permlane16_swap(b, b, false, false);
  return __builtin_bit_cast(float, (int)r[0]) +
         __builtin_bit_cast(float, (int)r[1]);
}
__device__ __forceinline__ float pair32_sum(float x) {
  const int b = __builtin_bit_cast(int, x);
  const auto r = __builtin_amdgcn_permlane32_swap(b, b, false, false);
  return __builtin_bit_cast(float, (int)r[0]) +
         __builtin_bit_cast(float, (int)r[1]);
}

constexpr int kBufferWord3 = 0x00020000;  // gfx9-family raw buffer format
// Cache policy of the K/V loads: non-temporal (each byte is read once).
constexpr int kLoadNT = 2;

__device__ __forceinline__ uint4 load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, kLoadNT);
  return make_uint4(x[0], x[1], x[2], x[3]);
}

// Per-lane byte offset of the loads, the same for every instruction: lane l
// reads row l / LPR of its RPI-row group at dims 8*(l % LPR).
// row_bytes = n_kv_head * HD * 2.
template <int HD>
__device__ __forceinline__ uint32_t lane_offset(uint32_t row_bytes, int lane) {
  using Geo = MGeo<HD>;
  return (uint32_t)(lane / Geo::LPR) * row_bytes +
         16u * (uint32_t)(lane % Geo::LPR);
}

// Raw buffer view of rows [first, hi) of one (sequence, KV head) cache slice:
// based at row `first`, record limit at row hi, so loads of rows at or past hi
// return zeros in hardware and are never fetched. Base and limit are
// wave-uniform (scalar registers).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_view(
    const uint16_t *seq, uint32_t row_bytes, uint32_t first, uint32_t hi) {
  const int limit = first < hi ? (int)((hi - first) * row_bytes) : 0;
  return __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t *>(seq + (size_t)first * (row_bytes / 2)), (short)0,
      limit, kBufferWord3);
}

// Workgroup barrier that orders LDS accesses only (no wait for outstanding
// global loads).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// s_waitcnt immediate for "at most n vector memory loads outstanding" (gfx9
// encoding: vmcnt in bits 3:0 and 15:14; expcnt and lgkmcnt left at their
// maxima, i.e. not waited for).
constexpr int vmcnt_imm(int n) {
  return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8);
}

// Eight fp32 values as eight fp16 bit patterns (v_cvt_f16_f32: round to
// nearest even, overflow to infinity), packed in element order.
__device__ __forceinline__ uint32_t f16x2_bits(float lo, float hi) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)lo) |
         ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)hi) << 16);
}
__device__ __forceinline__ uint4 f16x8(const float4v &x, const float4v &y) {
  return make_uint4(f16x2_bits(x[0], x[1]), f16x2_bits(x[2], x[3]),
                    f16x2_bits(y[0], y[1]), f16x2_bits(y[2], y[3]));
}

// Issue the loads of one tensor's rows of the 16-row tile starting at row tb
// (tb < hi).
template <int HD>
__device__ __forceinline__ void load_rows(uint4 (&x)[MGeo<HD>::NL],
                                          const uint16_t *seq,
                                          uint32_t row_bytes, uint32_t tb,
                                          uint32_t hi, uint32_t off) {
  using Geo = MGeo<HD>;
  // tb and hi are wave-uniform; without the explicit scalar copies the
  // compiler kept the loop's row counter in a vector register and wrapped
  // every load in a loop over distinct descriptors
  tb = __builtin_amdgcn_readfirstlane(tb);
  hi = __builtin_amdgcn_readfirstlane(hi);
#pragma unroll
  for (int i = 0; i < Geo::NL; ++i)
    x[i] = load16(rows_view(seq, row_bytes, tb + (uint32_t)(Geo::RPI * i), hi), off);
}

// Issue the loads of the 16-row tile starting at row tb (tb < hi): all K
// first (the scores need only K, and loads return in order), then V.
template <int HD>
__device__ __forceinline__ void load_tile(TileRegs<HD> &t, const uint16_t *kseq,
                                          const uint16_t *vseq,
                                          uint32_t row_bytes, uint32_t tb,
                                          uint32_t hi, uint32_t off) {
  load_rows<HD>(t.k, kseq, row_bytes, tb, hi, off);
  load_rows<HD>(t.v, vseq, row_bytes, tb, hi, off);
}

// Write a loaded tile's K (or V) rows into the wave's LDS slice, row-major
// with a pitch of STR bytes. The fences order these writes after the
// previous reads of the same bytes.
template <int HD, int STR>
__device__ __forceinline__ void stage_rows(const uint4 (&x)[MGeo<HD>::NL],
                                           unsigned char *dst, int lane) {
  using Geo = MGeo<HD>;
  wave_lds_fence();
#pragma unroll
  for (int i = 0; i < Geo::NL; ++i)
    *reinterpret_cast<uint4 *>(dst + (Geo::RPI * i + lane / Geo::LPR) * STR +
                               16 * (lane % Geo::LPR)) = x[i];
  wave_lds_fence();
}

// Several query rows per workgroup: the V rows of this tile from mask_from on
// are live for some columns only (the later query rows). The shared product
// O += Vᵀ·P would give every other column 0·v for them: exactly 0 for a
// finite v, but NaN where v is inf or NaN, while the causal mask leaves such a
// row out of an earlier query row entirely. So in a tile that holds such rows
// (rows j0 .. j1 - 1 of the tile, from mask_from to the workgroup's end row)
// they are kept out of the product: stash_masked_rows copies them into the
// wave's K area (free once the scores are computed; rows of 2*HD bytes) and
// zeroes them in the staged V, and after the product add_masked_rows adds p·v
// on the vector ALU for each lane's own column where the row is live
// (tb + j < lim). Only the tiles that hold a block's newest rows take this
// path, and only when those rows hold an inf or NaN: for finite rows the
// product is already exact. The check reads the rows once from LDS (8q/8kv,
// 8 rows per block, 28 layers: 8.33 against 9.64 us per layer at 2K, 18.2
// against 19.0 at 16K with the path always taken; the vector-ALU adds of up
// to 7 rows are the cost it saves). (Measured alternatives: the vector-ALU
// step between staging and product raised the several-row kernels'
// registers by ~30; writing the zeros and the copy while staging cost more
// than the path itself.)
struct MaskedRows {
  uint32_t j0, j1;
};

__device__ __forceinline__ MaskedRows masked_rows(uint32_t tb, uint32_t mask_from,
                                                  uint32_t row_end) {
  MaskedRows m;
  m.j0 = mask_from > tb ? mask_from - tb : 0u;
  m.j1 = row_end - tb < (uint32_t)kTileRows ? row_end - tb : (uint32_t)kTileRows;
  return m;
}

// Whether rows j0 .. j1 - 1 of the staged V hold an fp16 inf or NaN (an
// exponent of all ones), for the whole wave. Per 32-bit word: with the two
// exponent fields masked, adding 0x0400 to each carries into its half's sign
// bit exactly when the field is all ones.
template <int HD>
__device__ __forceinline__ bool masked_rows_nonfinite(const unsigned char *vlds,
                                                      MaskedRows m, int lane) {
  using Geo = MGeo<HD>;
  constexpr int CPR = HD / 8;  // 16-byte chunks per row
  const int n = (int)(m.j1 - m.j0) * CPR;
  uint32_t bad = 0;
  for (int c = lane; c < n; c += 64) {
    const uint4 w = *reinterpret_cast<const uint4 *>(
        vlds + (m.j0 + (uint32_t)(c / CPR)) * Geo::VSTR + (c % CPR) * 16);
    bad |= ((w.x & 0x7C007C00u) + 0x04000400u) & 0x80008000u;
    bad |= ((w.y & 0x7C007C00u) + 0x04000400u) & 0x80008000u;
    bad |= ((w.z & 0x7C007C00u) + 0x04000400u) & 0x80008000u;
    bad |= ((w.w & 0x7C007C00u) + 0x04000400u) & 0x80008000u;
  }
  return __builtin_amdgcn_ballot_w64(bad != 0u) != 0u;
}

template <int HD>
__device__ __forceinline__ void stash_masked_rows(unsigned char *vlds,
                                                  unsigned char *klds,
                                                  MaskedRows m, int lane) {
  using Geo = MGeo<HD>;
  constexpr int CPR = HD / 8;  // 16-byte chunks per row
  const int n = (int)(m.j1 - m.j0) * CPR;
  for (int c = lane; c < n; c += 64) {
    const uint32_t j = m.j0 + (uint32_t)(c / CPR);
    uint4 *src = reinterpret_cast<uint4 *>(vlds + j * Geo::VSTR + (c % CPR) * 16);
    *reinterpret_cast<uint4 *>(klds + (j - m.j0) * (2 * HD) + (c % CPR) * 16) = *src;
    *src = uint4{0u, 0u, 0u, 0u};
  }
}

// Lane (grp, col) holds dims 16b + 4grp + 0..3 of column col (the layout of
// the product's accumulators); p of row j and column col sits in lane
// 16 (j / 4) + col, entry j % 4. With one column block the lo-part lanes
// (col >= 8) hold the same column as lane col - 8, so only the hi-part lanes
// add; with two blocks every lane adds into the hi-part block.
template <int HD, int CB>
__device__ __forceinline__ void add_masked_rows(
    const unsigned char *klds, MaskedRows m, uint32_t tb, uint32_t lim,
    const float (&pv)[4], float4v (&oacc)[CB][MGeo<HD>::DB], int col, int grp,
    bool hi_col) {
  using Geo = MGeo<HD>;
  const bool adds = (CB == 2) || hi_col;
  for (uint32_t j = m.j0; j < m.j1; ++j) {
    const uint32_t k = j % 4;
    const float pk = k == 0 ? pv[0] : k == 1 ? pv[1] : k == 2 ? pv[2] : pv[3];
    const float p = __shfl(pk, (int)(16 * (j / 4)) + col);
    if (adds && tb + j < lim) {
#pragma unroll
      for (int b = 0; b < Geo::DB; ++b) {
        const half4 v4 = *reinterpret_cast<const half4 *>(
            klds + (j - m.j0) * (2 * HD) + (16 * b + 4 * grp) * 2);
#pragma unroll
        for (int i = 0; i < 4; ++i)
          oacc[0][b][i] = __builtin_fmaf(p, (float)v4[i], oacc[0][b][i]);
      }
    }
  }
}

// a4 + a5 for the loaded tile starting at row tb. mask_from: wave-uniform row
// from which some column may be masked; row_end: the workgroup's end row (no
// column sees a row past it); lim: this lane's column's end row (equal to
// mask_from with one query row per workgroup). SAFE: a column may
// have no live row yet (several query rows per workgroup), so -inf maxima are
// guarded. K is staged first and V only after the softmax, so the V rows
// (which arrive last) are written while the exponentials run.
// CB = 1: one 16-column MFMA block, hi parts in columns 0..7 and lo parts in
// 8..15 (added by a DPP rotation). CB = 2: two blocks of 16 columns, block 0
// the hi parts and block 1 the lo parts of 16 (row, head) columns (added
// lane by lane); every product then runs twice.
// after_k / after_v run right after the tile's K / V rows have been staged
// (their registers are free from then on): the loop uses them to issue the
// next tile's loads early where that measured faster.
template <int HD, bool SAFE, int CB, typename AfterK, typename AfterV>
__device__ __forceinline__ void compute_tile(
    TileRegs<HD> &t, AfterK after_k, AfterV after_v, unsigned char *slice,
    uint32_t tb,
    uint32_t mask_from, uint32_t row_end, uint32_t lim,
    const half8 (&qf)[CB][MGeo<HD>::KS],
    float4v (&oacc)[CB][MGeo<HD>::DB], float &m_run, float &m_true,
    float &s_run, int col, int grp, int lane, bool hi_col) {
  using Geo = MGeo<HD>;
  unsigned char *vlds = slice + Geo::KTILE;
  // Raised issue priority while a landed tile is computed: the wave's next
  // loads wait for this compute (28 layers at 32K rows: 16.37 against 16.45
  // us per layer without it).
  __builtin_amdgcn_s_setprio(2);
  // a4: scores S = K · Q'ᵀ, K operands read back from the staged rows.
  stage_rows<HD, Geo::KSTR>(t.k, slice, lane);
  after_k(t);
  uint4 ka[Geo::KS];
#pragma unroll
  for (int ks = 0; ks < Geo::KS; ++ks)
    ka[ks] = *reinterpret_cast<const uint4 *>(slice + col * Geo::KSTR +
                                               64 * ks + 16 * grp);
  // two accumulators (even and odd k-steps) halve the dependent MFMA chain
  // (28 layers at 32K rows: partial kernel 13.15 against 13.3 us)
  float4v sc[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    float4v s0 = float4v{0.f, 0.f, 0.f, 0.f};
    float4v s1 = float4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < Geo::KS; ks += 2) {
      s0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_half8(ka[ks]),
                                                  qf[cb][ks], s0, 0, 0, 0);
      if (ks + 1 < Geo::KS)
        s1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(
            as_half8(ka[ks + 1]), qf[cb][ks + 1], s1, 0, 0, 0);
    }
    sc[cb] = s0 + s1;
  }
  // hi + lo columns; rows at or past the column's end (last tiles only) score
  // -inf.
  float s[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    if constexpr (CB == 1)
      s[r] = add_ror8(sc[0][r]);
    else
      s[r] = sc[0][r] + sc[1][r];
  }
  if (tb + kTileRows > mask_from) {
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (tb + (uint32_t)(4 * grp + r) >= lim) s[r] = neg_inf();
  }
  float mt = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
  mt = pair32_max(pair16_max(mt));
  // a5: online softmax against a reference max m_run that moves only when a
  // tile's max exceeds it by more than kLazyLog2 (and always from -inf; the
  // tile's first row is live, so mt is finite). Until then p = exp2(s - m_run)
  // may exceed 1, up to 2^kLazyLog2, which the fp32 sums and the fp16 hi + lo
  // split of p carry at full precision; the rescale of the accumulators is
  // skipped for most tiles. The exact running max m_true is kept beside it,
  // and the final merge takes every state to m_true, so the records are the
  // same (max, sum, output) triple as with an exact max at every tile.
  m_true = fmaxf(m_true, mt);
  const float mn = (mt > m_run + kLazyLog2) ? mt : m_run;
  // 0 while m_run is -inf (and with SAFE also while mn still is)
  const float corr = (SAFE && m_run == neg_inf()) ? 0.0f : fast_exp2(m_run - mn);
  const float mref = (SAFE && mn == neg_inf()) ? 0.0f : mn;
  // p hi and lo parts in this lane's rows: the B operands of O += Vᵀ·P
  half4 pf[CB];
  float pv[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const float p = fast_exp2(s[r] - mref);  // exp2(-inf) = 0
    pv[r] = p;
    const _Float16 h = (_Float16)p;
    if constexpr (CB == 1) {
      pf[0][r] = hi_col ? h : (_Float16)(p - (float)h);
    } else {
      pf[0][r] = h;
      pf[1][r] = (_Float16)(p - (float)h);
    }
  }
  const float psum = (pv[0] + pv[1]) + (pv[2] + pv[3]);
  // Rescale only when some column's reference moved (else corr is 1 for
  // every column and the products would change nothing).
  if (__any(mn != m_run)) {
    s_run *= corr;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
      for (int b = 0; b < Geo::DB; ++b) oacc[cb][b] *= corr;
  }
  s_run += psum;
  m_run = mn;

  // O += Vᵀ · P: lane (grp, col) reads dim 16b + col of rows 4*grp + 0..3,
  // the same row order as its p values.
  stage_rows<HD, Geo::VSTR>(t.v, vlds, lane);
  after_v(t);
  const MaskedRows mr = masked_rows(tb, mask_from, row_end);
  // Only an inf or NaN among those rows must stay out of the product: a
  // finite row is multiplied by exactly p = 0 in the columns that cannot
  // see it.
  bool split_rows = SAFE && tb + kTileRows > mask_from && mask_from < row_end;
  if (split_rows) split_rows = masked_rows_nonfinite<HD>(vlds, mr, lane);
  if (split_rows) stash_masked_rows<HD>(vlds, slice, mr, lane);
  const int c4 = col >> 2;
  const int cm = col & 3;
#pragma unroll
  for (int b = 0; b < Geo::DB; ++b) {
    // (C-style cast: address-space conversion of the generic LDS pointer)
    lds_short4v *a0 = (lds_short4v *)(vlds + (4 * grp + c4) * Geo::VSTR +
                                      (16 * b + 4 * cm) * 2);
    const short4v r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(a0);
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
      oacc[cb][b] = __builtin_amdgcn_mfma_f32_16x16x16f16(
          __builtin_bit_cast(half4, r0), pf[cb], oacc[cb][b], 0, 0, 0);
  }
  if (split_rows)
    add_masked_rows<HD, CB>(slice, mr, tb, lim, pv, oacc, col, grp, hi_col);
  __builtin_amdgcn_s_setprio(0);
}

// A column's output: hi part + lo part. One block: this lane's column plus
// the column 8 lanes along (a DPP rotation; every lane of the wave must be
// active); two blocks: the same lane's entries of both.
template <int CB, int DB>
__device__ __forceinline__ float hilo_sum(const float4v (&oacc)[CB][DB], int i,
                                          int r) {
  if constexpr (CB == 1)
    return add_ror8(oacc[0][i][r]);
  else
    return oacc[0][i][r] + oacc[1][i][r];
}

// PER_HEAD = false: one workgroup per (split, KV head, sequence) computes all
// G query heads of the group (blockIdx.y = KV head). PER_HEAD = true (with
// G = 1): one workgroup per (split, query head, sequence), blockIdx.y = query
// head, reading KV head blockIdx.y / a.kv_group -- the per-query-head grid,
// kept as an A/B baseline; every KV row is then read once per query head.
// R: query rows per workgroup (several query rows per sequence). The MFMA
// columns then hold (row, head) pairs, column c = r * G + g, so every K/V row
// is read once for the R rows; with R = 1 each workgroup serves one row.
// FOLD: the decode-step form with the KV-cache append folded in (one query
// row, grouped); a separate instantiation, so that the plain forms keep
// their register count.
template <int HD, int G, bool PER_HEAD = false, int R = 1, bool FOLD = false>
__global__ __launch_bounds__(MWaves<HD>::kThr, MWaves<HD>::W == 8 ? 1 : 2) void
partial_mfma_kernel(PartialArgs a) {
  using Geo = MGeo<HD>;
  constexpr int kW = MWaves<HD>::W;       // waves per workgroup
  constexpr int kT = MWaves<HD>::kThr;    // threads per workgroup
  constexpr int SLICE = Geo::SLICE;
  constexpr int NC = G * R;                          // (row, head) columns
  // one 16-column block holds 8 columns (hi and lo parts), two hold 16
  constexpr int CB = NC > 8 ? 2 : 1;
  static_assert(G >= 1 && G <= 8 && NC <= 16, "group x rows");
  static_assert(CB == 1 || HD <= 128, "two column blocks: hd 64 and 128");
  static_assert(!PER_HEAD || (G == 1 && R == 1), "per-head form: one head");
  static_assert(!FOLD || (!PER_HEAD && R == 1), "folded append: one row");
  // split, first query head / G, and (sequence, first query row of this
  // workgroup)
  int sp_ = blockIdx.x;
  int hy_ = blockIdx.y;
  detail::RowSel rs;
  if (a.pair_rows) {
    // grid dim3(8 * row blocks, n_splits / 8, n_kv_head * batch): the row
    // blocks of one (split, KV head, sequence) are 8 apart in the dispatch
    // order, which deals workgroups to the XCDs in turn, so they run on one
    // XCD at the same time and the later reads of each K/V tile are served
    // by its L2
    sp_ = (int)(blockIdx.x & 7u) + 8 * (int)blockIdx.y;
    rs.b = blockIdx.z / a.n_kv_head;
    hy_ = blockIdx.z - rs.b * a.n_kv_head;
    rs.t = (int)(blockIdx.x >> 3) * R;
  } else if constexpr (R == 1) {
    rs = detail::row_sel(a);
  } else {
    const int nrb = (a.n_q + R - 1) / R;
    rs.b = blockIdx.z / nrb;
    rs.t = (blockIdx.z - rs.b * nrb) * R;
  }
  const int sp = sp_;
  const int hy = hy_;
  const int hk = PER_HEAD ? hy / a.kv_group : hy;    // KV head
  const int b = rs.b;
  const int tid = threadIdx.x;
  // wave index, provably uniform (scalar) so per-tile row math stays scalar
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int col = lane & 15;
  const int grp = lane >> 4;
  const bool hi_col = col < 8;   // (one column block) hi part of a column

  __shared__ __attribute__((aligned(16))) unsigned char sm_v[kW * SLICE];
  // each wave's state per column: (reference max, exact max, sum, unused)
  __shared__ float4 sm_st[kW][NC];
  // the query operand, converted once per workgroup (lane-major per ks)
  __shared__ half8 sm_q[CB][Geo::KS][64];
  // a column's output in the wave's slice: HD floats padded by 4, so that
  // column c starts 4c banks along and the 16-byte writes of the (up to 16)
  // columns of one row group fall in distinct banks. (A pad of 16 floats,
  // used before, put columns 0, 2, 4, 6 of one column block on the same banks:
  // 2- to 4-way conflicts; the pad of 4 measured 7.35 against 7.49 us for the
  // partial kernel at head_dim 256, 8,400 rows, and 0.02-0.06 us faster at
  // head_dim 128.)
  constexpr int OSTR = (HD + 4) * 4;
  static_assert(NC * OSTR <= SLICE, "output state fits the wave's slice");

  // This lane's MFMA column: (row, head) pair c = r * G + g of the
  // workgroup's rows (column col % 8 in one block, col in two).
  const int gq = CB == 1 ? (col & 7) : col;          // this lane's column
  bool col_valid;                                    // column maps to a row
  int col_t, col_g;                                  // and its (row, head)
  if constexpr (R == 1) {
    col_valid = gq < G;
    col_t = rs.t;
    col_g = gq < G ? gq : 0;
  } else {
    const int r_c = gq / G;
    col_valid = gq < NC && rs.t + r_c < a.n_q;
    col_t = col_valid ? rs.t + r_c : rs.t;
    col_g = col_valid ? gq - r_c * G : 0;
  }

  // a1: the live length's read is issued first; its latency (it queues
  // behind other workgroups' K/V loads) overlaps the query loads below.
  const int pos_b = a.positions[b];

  // a3: the queries do not depend on the live length, so wave 0 issues their
  // loads while the live length is in flight (the other waves take the
  // converted operand from LDS, below). Lane (grp, col) loads dims 32*ks + 8*grp .. +7
  // of column col's (row, head).
  float4 qraw[Geo::KS][2];
  if (wave == 0) {
    const detail::RowSel qs{b, col_t};
    const float *qrow =
        a.q + detail::q_offset(a, qs, hy * G + col_g, HD) + 8 * grp;
#pragma unroll
    for (int ks = 0; ks < Geo::KS; ++ks) {
      qraw[ks][0] = *reinterpret_cast<const float4 *>(qrow + 32 * ks);
      qraw[ks][1] = *reinterpret_cast<const float4 *>(qrow + 32 * ks + 4);
    }
  }

  // a1 + a2: live length and this split's rows; with several query rows,
  // a row's rows end at min(hi, its own live length). The waves run to the
  // end of the workgroup's last row; masking starts at its first row's end,
  // and each column stops at its own row's end.
  const detail::SplitRange rg = detail::split_range_at(a, sp, pos_b);
  const long long lo = rg.lo;
  long long hi, mask_from, col_end;
  if constexpr (R == 1) {
    hi = a.n_q == 1 ? rg.hi : detail::row_end_pos(a, pos_b, rs.t, rg.hi);
    mask_from = hi;
    col_end = hi;
  } else {
    const int t_last = min(rs.t + R - 1, a.n_q - 1);
    hi = detail::row_end_pos(a, pos_b, t_last, rg.hi);
    mask_from = detail::row_end_pos(a, pos_b, rs.t, rg.hi);
    col_end = col_valid ? detail::row_end_pos(a, pos_b, col_t, rg.hi) : hi;
  }

  // This (sequence, KV head) slice of the caches: row r at byte r * row_bytes.
  const uint32_t row_bytes = (uint32_t)(a.n_kv_head * HD * 2);
  const size_t seq_base = ((size_t)b * (size_t)a.max_ctx * a.n_kv_head + hk) * HD;
  const uint16_t *kseq = a.k + seq_base;
  const uint16_t *vseq = a.v + seq_base;
  const uint32_t off = lane_offset<HD>(row_bytes, lane);
  unsigned char *slice = sm_v + wave * SLICE;
  const uint32_t hi32 = (uint32_t)hi;
  const uint32_t mask32 = (uint32_t)mask_from;
  const uint32_t lim32 = (uint32_t)col_end;
  const uint32_t step = (uint32_t)(kW * kTileRows);
  uint32_t t0 = (uint32_t)lo + (uint32_t)(wave * kTileRows);
  if (lo >= hi) t0 = hi32;  // idle split

  // Folded append (a decode step with one query row): this sequence's new
  // row for this KV head goes to position pos_b. The wave whose tile holds
  // that position issues the new row's loads now; on reaching the tile it
  // writes the row into the caches and uses the converted values in place of
  // the ones it loaded (the cache still held that row's previous contents).
  uint32_t app_tb = 0xFFFFFFFFu;    // start of the tile holding the new row
  float4v knew[2], vnew[2];         // this lane's 8 dims of it, fp32
  if constexpr (FOLD) {
    if (a.k_new != nullptr && pos_b >= 0 && pos_b < a.max_ctx &&
        (long long)pos_b >= lo && (long long)pos_b < hi) {
      const uint32_t j = ((uint32_t)pos_b - (uint32_t)lo) / kTileRows;
      if ((int)(j % kW) == wave) {
        app_tb = (uint32_t)lo + j * kTileRows;
        const size_t src =
            ((size_t)b * a.n_kv_head + hk) * HD + 8 * (lane % Geo::LPR);
        knew[0] = *reinterpret_cast<const float4v *>(a.k_new + src);
        knew[1] = *reinterpret_cast<const float4v *>(a.k_new + src + 4);
        vnew[0] = *reinterpret_cast<const float4v *>(a.v_new + src);
        vnew[1] = *reinterpret_cast<const float4v *>(a.v_new + src + 4);
      }
    }
  }
  auto put_new_row = [&](TileRegs<HD> &t) {
    const uint32_t r = (uint32_t)pos_b - app_tb;       // row in the tile
    const bool mine = (uint32_t)(lane / Geo::LPR) == r % Geo::RPI;
    // Pinned here: hoisted to where the loads are issued, the conversion
    // would make the wave wait for the new row before its first tile's loads.
    float4v k0 = knew[0], k1 = knew[1], v0 = vnew[0], v1 = vnew[1];
    asm volatile("" : "+v"(k0), "+v"(k1), "+v"(v0), "+v"(v1));
    const uint4 kh = f16x8(k0, k1);
    const uint4 vh = f16x8(v0, v1);
#pragma unroll
    for (int i = 0; i < Geo::NL; ++i) {
      if (i == (int)(r / Geo::RPI) && mine) {
        t.k[i] = kh;
        t.v[i] = vh;
      }
    }
    if (mine) {
      const size_t dst = ((size_t)b * a.max_ctx + (size_t)pos_b) *
                             (size_t)a.n_kv_head * HD +
                         (size_t)hk * HD + 8 * (lane % Geo::LPR);
      *reinterpret_cast<uint4 *>(a.k_app + dst) = kh;
      *reinterpret_cast<uint4 *>(a.v_app + dst) = vh;
    }
  };

  float4v oacc[CB][Geo::DB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb)
#pragma unroll
    for (int i = 0; i < Geo::DB; ++i) oacc[cb][i] = float4v{0.f, 0.f, 0.f, 0.f};
  float m_run = neg_inf();   // reference max (base-2 units), see compute_tile
  float m_true = neg_inf();  // exact running max
  float s_run = 0.0f;

  // B operand of S = K·Q'ᵀ, the same in every wave: with one block, column
  // col holds (row, head) col % 8, hi part in columns 0..7 and lo part in
  // 8..15; with two, block 0 holds the hi parts and block 1 the lo parts of
  // columns 0..15 (zero for unused columns); dims 32*ks + 8*grp + e,
  // pre-scaled to base-2 units.
  // Wave 0 converts it (its query loads come back while the first tile is in
  // flight) and hands it to the other waves through LDS: one query read per
  // workgroup instead of one per wave.
  auto share_q = [&] {
#pragma unroll
    for (int ks = 0; ks < Geo::KS; ++ks) {
      const float x[8] = {qraw[ks][0].x, qraw[ks][0].y, qraw[ks][0].z,
                          qraw[ks][0].w, qraw[ks][1].x, qraw[ks][1].y,
                          qraw[ks][1].z, qraw[ks][1].w};
      half8 h8, l8;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        // q' = q * scale_log2 as hi + lo: hi = fp16(q'), lo = fp16 of the
        // exact product minus hi (an explicit fma, so every instantiation
        // rounds the same way whatever the compiler contracts).
        const _Float16 h = (_Float16)(x[e] * a.scale_log2);
        const float lo = __builtin_fmaf(x[e], a.scale_log2, -(float)h);
        if constexpr (CB == 1) {
          const _Float16 val = hi_col ? h : (_Float16)lo;
          h8[e] = col_valid ? val : (_Float16)0.0f;
        } else {
          h8[e] = col_valid ? h : (_Float16)0.0f;
          l8[e] = col_valid ? (_Float16)lo : (_Float16)0.0f;
        }
      }
      sm_q[0][ks][lane] = h8;
      if constexpr (CB == 2) sm_q[1][ks][lane] = l8;
    }
  };
  // Wave 0 has the split's first tile, so when it has no rows no wave has and
  // nobody needs the operand. The busy and idle paths each pass the barrier
  // on their own (a workgroup barrier counts waves, not call sites; every
  // wave passes exactly one here), so that on the busy path the compiler's
  // load counters see the query loads as older than the tile's: the
  // conversion waits for the queries alone, and the first tile's waits are
  // not widened to cover query loads. A busy wave other than 0 issued no
  // query loads, and an idle wave 0 drains its unused ones; explicit waits
  // tell the counters so (with 2 * NL tile loads issued the first returns at
  // once). The barrier orders LDS only: the operand is the one thing shared.
  // A wave whose first tile starts at or past hi has no rows: it keeps the
  // empty state (-inf, 0, 0) and issues no K/V loads at all.
  const bool busy = t0 < hi32;
  if (busy) {
    TileRegs<HD> tr;
    load_tile<HD>(tr, kseq, vseq, row_bytes, t0, hi32, off);
    if (wave == 0)
      share_q();
    else
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * Geo::NL));
    lds_barrier();
    half8 qf[CB][Geo::KS];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
      for (int ks = 0; ks < Geo::KS; ++ks) qf[cb][ks] = sm_q[cb][ks][lane];

    // a4 + a5 over this wave's tiles: compute the landed tile (staged
    // through LDS), then issue the next tile's loads (only tiles with rows:
    // even loads past the record limit, which return zeros without touching
    // memory, cost address-unit time). Each wave has at most one tile in
    // flight: at 32K rows, issuing the next tile before computing the current
    // one (one more tile in flight per wave) measured 0.4 us per layer
    // slower and a second register tile 0.6 us, because deeper memory queues
    // serve the workgroups dispatched last later still; issuing the next
    // tile's K and V as soon as the current ones are staged (in a separate
    // code path, so that the load counters are exact) is within 0.1 us either
    // way at 2K-32K rows, and issuing only the second tile early is 0.3 us
    // slower at 16K and 32K. At head_dim 256 (few tiles per wave, each
    // computed for longer) the early issue measured faster (8,400 rows: 7.80
    // against 7.99 us). Written as below, with one path for both cases, the
    // compiler's counters make the V stage wait for the next tile's K loads
    // as well; the two-path form with exact counts was slower there (254
    // against 199 VGPRs; partial kernel 7.85 against 7.51 us at 8,400 rows,
    // 14.4 against 14.2 us at 32K).
    constexpr bool kEarly = HD >= 256;
    while (true) {
      if constexpr (FOLD) {
        if (t0 == app_tb) put_new_row(tr);
      }
      const uint32_t nt = t0 + step;
      const bool more = nt < hi32;
      compute_tile<HD, (R > 1), CB>(
          tr,
          [&](TileRegs<HD> &x) {
            if (kEarly && more) load_rows<HD>(x.k, kseq, row_bytes, nt, hi32, off);
          },
          [&](TileRegs<HD> &x) {
            if (kEarly && more) load_rows<HD>(x.v, vseq, row_bytes, nt, hi32, off);
          },
          slice, t0, mask32, hi32, lim32, qf, oacc, m_run, m_true, s_run, col,
          grp, lane, hi_col);
      t0 = nt;
      if (!more) break;
      if constexpr (!kEarly) load_tile<HD>(tr, kseq, vseq, row_bytes, t0, hi32, off);
    }
  } else {
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    lds_barrier();
  }

  // a6: merge the waves and write the records. Each wave puts its state
  // in LDS (reference max, exact max and sum per head; O with the hi and lo
  // columns added), then after one barrier every thread merges one float4 of
  // one head's output over the waves with weights exp2(m_ref - m_all),
  // m_all the largest exact max: the record is relative to the exact max.
  // This runs after the workgroup's last data has landed, so its latency is
  // on the kernel's critical path: all of a thread's LDS reads are issued
  // before any of the arithmetic.
  s_run = pair32_sum(pair16_sum(s_run));
  constexpr int D4 = HD / 4;
  // Output sums of column (row r, head g): oc0 + (r * n_head + g) * HD; its
  // header at hdr_offset(rs.b, rs.t + r, sp, hy * G + g).
  float *oc0 = a.partials + detail::oc_offset(a, rs, sp, hy * G, HD);

  // A split of at most one tile (short contexts over many splits), or an
  // idle one: only wave 0 can have rows, so it writes the records straight
  // from its registers, with the same arithmetic as the merge below when
  // waves 1..3 hold the empty state (weight 0, output 0; the "+ 0" is the
  // merge's fma with a zero weight, kept for identical signed zeros), and no
  // wave waits at a barrier.
  if ((uint32_t)lo + kTileRows >= hi32) {
    if (wave != 0) return;
    // hi + lo parts first, with every lane of the wave active (with one
    // column block the lo column lanes are the rotation's sources)
    float4v osum[Geo::DB];
#pragma unroll
    for (int i = 0; i < Geo::DB; ++i)
#pragma unroll
      for (int k = 0; k < 4; ++k) osum[i][k] = hilo_sum<CB>(oacc, i, k);
    if (col >= NC) return;
    const int r = col / G;
    if (R > 1 && rs.t + r >= a.n_q) return;
    const float c = (m_run == neg_inf()) ? 0.0f : fast_exp2(m_run - m_true);
    const int g = col - r * G;
    float *oc = oc0 + (size_t)(r * a.n_head + g) * HD;
#pragma unroll
    for (int i = 0; i < Geo::DB; ++i) {
      float4 o;
      o.x = fmaf(c, osum[i][0], 0.0f) + 0.0f;
      o.y = fmaf(c, osum[i][1], 0.0f) + 0.0f;
      o.z = fmaf(c, osum[i][2], 0.0f) + 0.0f;
      o.w = fmaf(c, osum[i][3], 0.0f) + 0.0f;
      *reinterpret_cast<float4 *>(oc + 16 * i + 4 * grp) = o;
    }
    if (grp == 0)
      *reinterpret_cast<float4 *>(
          a.headers + detail::hdr_offset(a, rs.b, rs.t + r, sp, hy * G + g)) =
          make_float4(m_true * detail::kLn2, fmaf(c, s_run, 0.0f) + 0.0f,
                      __builtin_bit_cast(float, (int32_t)rg.lo),
                      __builtin_bit_cast(float, (int32_t)rg.hi));
    return;
  }

  if (grp == 0 && col < NC) sm_st[wave][col] = make_float4(m_run, m_true, s_run, 0.f);
  wave_lds_fence();  // the slice's last tile reads come first
#pragma unroll
  for (int i = 0; i < Geo::DB; ++i) {
    float o4[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) o4[r] = hilo_sum<CB>(oacc, i, r);
    if (col < NC)
      *reinterpret_cast<float4 *>(slice + col * OSTR + (16 * i + 4 * grp) * 4) =
          make_float4(o4[0], o4[1], o4[2], o4[3]);
  }
  __syncthreads();
  for (int idx = tid; idx < NC * D4; idx += kT) {
    const int gg = idx / D4;
    const int d4 = idx % D4;
    // column gg = (row r, head g); rows past n_q have no record
    const int r = gg / G;
    if (R > 1 && rs.t + r >= a.n_q) continue;
    float4 stw[kW], x[kW];
#pragma unroll
    for (int w = 0; w < kW; ++w) {
      stw[w] = sm_st[w][gg];
      x[w] = *reinterpret_cast<const float4 *>(sm_v + w * SLICE + gg * OSTR +
                                               16 * d4);
    }
    float mm = neg_inf();
#pragma unroll
    for (int w = 0; w < kW; ++w) mm = fmaxf(mm, stw[w].y);
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    float st = 0.0f;
#pragma unroll
    for (int w = 0; w < kW; ++w) {
      const float mw = stw[w].x;
      const float c = (mw == neg_inf()) ? 0.0f : fast_exp2(mw - mm);
      acc.x = fmaf(c, x[w].x, acc.x);
      acc.y = fmaf(c, x[w].y, acc.y);
      acc.z = fmaf(c, x[w].z, acc.z);
      acc.w = fmaf(c, x[w].w, acc.w);
      st = fmaf(c, stw[w].z, st);
    }
    const int g = gg - r * G;  // row t + r: n_head record heads on
    *reinterpret_cast<float4 *>(oc0 + (size_t)(r * a.n_head + g) * HD +
                                4 * d4) = acc;
    if (d4 == 0)
      *reinterpret_cast<float4 *>(
          a.headers + detail::hdr_offset(a, rs.b, rs.t + r, sp, hy * G + g)) =
          make_float4(mm * detail::kLn2, st,
                      __builtin_bit_cast(float, (int32_t)rg.lo),
                      __builtin_bit_cast(float, (int32_t)rg.hi));
  }
}

// Grid of the grouped kernel with `blocks` workgroups (blocks of query rows)
// per (split, KV head, sequence). With more than one, the blocks of one split
// read the same K/V rows, and the paired grid runs them side by side on one
// XCD (at 32K rows, 28q/4kv hd128, 4 rows: 21.5 against 24.9 us per layer
// with the plain grid); it needs a split count that is a multiple of 8.
PartialArgs with_row_grid(const PartialArgs &args, int blocks, int batch,
                          dim3 &grid) {
  PartialArgs a = args;
  a.pair_rows = blocks > 1 && a.n_splits % 8 == 0 &&
                (long long)a.n_kv_head * batch <= 65535;
  grid = a.pair_rows ? dim3(8 * blocks, a.n_splits / 8, a.n_kv_head * batch)
                     : dim3(a.n_splits, a.n_kv_head, batch * blocks);
  return a;
}

template <int HD, int G>
hipError_t launch_one(const PartialArgs &a, int batch, hipStream_t stream) {
  if (a.k_new != nullptr) {
    hipLaunchKernelGGL((partial_mfma_kernel<HD, G, false, 1, true>),
                       dim3(a.n_splits, a.n_kv_head, batch), dim3(MWaves<HD>::kThr),
                       0, stream, a);
  } else {
    dim3 grid;
    const PartialArgs b = with_row_grid(a, a.n_q, batch, grid);
    hipLaunchKernelGGL((partial_mfma_kernel<HD, G>), grid, dim3(MWaves<HD>::kThr), 0,
                       stream, b);
  }
  return hipGetLastError();
}

template <int HD>
hipError_t launch_hd(int group, const PartialArgs &a, int batch,
                     hipStream_t stream) {
  switch (group) {
    case 1: return launch_one<HD, 1>(a, batch, stream);
    case 2: return launch_one<HD, 2>(a, batch, stream);
    case 3: return launch_one<HD, 3>(a, batch, stream);
    case 4: return launch_one<HD, 4>(a, batch, stream);
    case 5: return launch_one<HD, 5>(a, batch, stream);
    case 6: return launch_one<HD, 6>(a, batch, stream);
    case 7: return launch_one<HD, 7>(a, batch, stream);
    case 8: return launch_one<HD, 8>(a, batch, stream);
    default: return hipErrorInvalidValue;
  }
}

template <int HD, int G, int R>
hipError_t launch_rows(const PartialArgs &a, int batch, hipStream_t stream) {
  dim3 grid;
  const PartialArgs b = with_row_grid(a, (a.n_q + R - 1) / R, batch, grid);
  hipLaunchKernelGGL((partial_mfma_kernel<HD, G, false, R>), grid,
                     dim3(MWaves<HD>::kThr), 0, stream, b);
  return hipGetLastError();
}

template <int HD>
hipError_t launch_rows_hd(int group, int rows, const PartialArgs &a,
                          int batch, hipStream_t stream) {
  switch (group * 16 + rows) {
    case 1 * 16 + 2: return launch_rows<HD, 1, 2>(a, batch, stream);
    case 1 * 16 + 4: return launch_rows<HD, 1, 4>(a, batch, stream);
    case 1 * 16 + 8: return launch_rows<HD, 1, 8>(a, batch, stream);
    case 2 * 16 + 2: return launch_rows<HD, 2, 2>(a, batch, stream);
    case 2 * 16 + 4: return launch_rows<HD, 2, 4>(a, batch, stream);
    case 3 * 16 + 2: return launch_rows<HD, 3, 2>(a, batch, stream);
    case 4 * 16 + 2: return launch_rows<HD, 4, 2>(a, batch, stream);
    default: break;
  }
  if constexpr (HD <= 128) {
    // two column blocks
    switch (group * 16 + rows) {
      case 2 * 16 + 8: return launch_rows<HD, 2, 8>(a, batch, stream);
      case 3 * 16 + 4: return launch_rows<HD, 3, 4>(a, batch, stream);
      case 4 * 16 + 4: return launch_rows<HD, 4, 4>(a, batch, stream);
      case 5 * 16 + 2: return launch_rows<HD, 5, 2>(a, batch, stream);
      case 6 * 16 + 2: return launch_rows<HD, 6, 2>(a, batch, stream);
      case 7 * 16 + 2: return launch_rows<HD, 7, 2>(a, batch, stream);
      case 8 * 16 + 2: return launch_rows<HD, 8, 2>(a, batch, stream);
      default: break;
    }
  }
  return hipErrorInvalidValue;
}

template <int HD>
hipError_t launch_per_head(const PartialArgs &a, int batch, hipStream_t stream) {
  hipLaunchKernelGGL((partial_mfma_kernel<HD, 1, true>),
                     dim3(a.n_splits, a.n_head, batch), dim3(MWaves<HD>::kThr), 0,
                     stream, a);
  return hipGetLastError();
}

}  // namespace

// Query rows per workgroup for n_q rows at group size G, R in {1, 2, 4, 8}:
// as many as the MFMA columns hold -- one 16-column block holds G * R <= 8
// (hi and lo parts side by side), two blocks hold G * R <= 16 (hd 64 and
// 128 only) -- and no more than the smallest such R that covers n_q.
int rows_per_workgroup(int head_dim, int group, int n_q) {
  if (n_q <= 1) return 1;
  const bool two = head_dim <= 128;
  const int cap = group == 1   ? 8
                  : group == 2 ? (two ? 8 : 4)
                  : group <= 4 ? (two ? 4 : 2)
                  : two ? 2 : 1;
  int r = 1;
  while (r < cap && r < n_q) r *= 2;
  return r;
}

hipError_t launch_partial_per_head(int head_dim, const PartialArgs &a,
                                   int batch, hipStream_t stream) {
  switch (head_dim) {
    case 64: return launch_per_head<64>(a, batch, stream);
    case 128: return launch_per_head<128>(a, batch, stream);
    case 256: return launch_per_head<256>(a, batch, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_partial_mfma(int head_dim, int group, const PartialArgs &a,
                               int batch, hipStream_t stream) {
  const int rows = rows_per_workgroup(head_dim, group, a.n_q);
  if (rows > 1) {
    switch (head_dim) {
      case 64: return launch_rows_hd<64>(group, rows, a, batch, stream);
      case 128: return launch_rows_hd<128>(group, rows, a, batch, stream);
      case 256: return launch_rows_hd<256>(group, rows, a, batch, stream);
      default: return hipErrorInvalidValue;
    }
  }
  switch (head_dim) {
    case 64: return launch_hd<64>(group, a, batch, stream);
    case 128: return launch_hd<128>(group, a, batch, stream);
    case 256: return launch_hd<256>(group, a, batch, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace splitkv
