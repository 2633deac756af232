// Batched row GEMMs on the gfx950 matrix cores: stage-1 centroid scores
// (bf16, INT4 or INT8 centroids), the dense head and the dense pass of the
// speculative verification for batches of bf16 queries, with
// v_mfma_f32_16x16x32_bf16 tiles (16 rows x 16 queries x 32 elements of d per
// instruction, fp32 accumulation); and the cluster-major stage 2.
//
// Sources (page title and section): FlashHead technical explainer
// (framerc.cn) §1.1 (dense head), §1.2.2 (stage-1 scores), §1.2.4 and §2.3
// (INT4 g32 centroids, bf16 tokens); "FlashHead: Efficient Drop-In
// Replacement for the Classification Head in Language Model Inference"
// (arXiv 2603.14591), abstract.
//
// Operand layout of the instruction (checked on the device): lane l holds
// A's row l % 16 and B's column l % 16 at k = 8 (l / 16) .. + 7, and the
// result's column l % 16 at rows 4 (l / 16) .. + 3.
//
// Tiling: a workgroup is 4 waves; wave w owns MT row tiles of 16 (rows
// [64 MT x + 16 MT w, +16 MT)) and all NT query tiles of 16 of the grid row
// y, so one workgroup covers 64 MT rows x 16 NT queries.  d is walked in
// blocks of 128 elements: the queries' block of h is staged in LDS (double
// buffered, the next block's loads in flight during the current block's
// products) and shared by the 4 waves; each wave's rows stream from HBM
// straight into registers, also one block ahead.  With B <= 128 queries in
// one grid row, every row of E or C is read from HBM once per call.
//
// bf16 rows: MFMA step s of block blk takes elements 128 blk + 32 s .. + 31,
// lane group g (g = l / 16) holding 8 g .. + 7 of them, for both operands:
// one load instruction then reads one contiguous 64-byte run per row.  (With
// lane group g owning 64 contiguous bytes across the steps, an instruction
// touched four sectors per row; that order was 5-7% slower on the dense head
// and the cluster-major stage 2.)
//
// INT4 rows (the defined value sum_g sigma[k, g] sum_{i in g} q h): one MFMA
// step is exactly one 32-element group.  The packed nibbles are re-laid out
// at create (fh_engine) so that lane group g's four-byte share of four
// consecutive groups is one 16-byte load.  A nibble q becomes the bf16 value
// 136 + q (bit pattern 0x4300 | (q + 8), exact), and a second MFMA with the
// constant -136 removes the offset, so the tile holds sum q h exactly up to
// fp32 rounding; the group's fp16 scales then scale it into the running
// score with one FMA per element.
#include <algorithm>
#include <cmath>
#include <type_traits>

#include "fh_blocks.hpp"

namespace fh {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// A 16-byte load with the non-temporal hint, for the bf16 operand streams
// read in order (the fragment-order copies of C and E).  Gathered rows and
// the INT4 codes keep ordinary loads: the hint measured slower on both.
__device__ __forceinline__ uint4 ld_stream(const void* p) {
  const u32x4 v = __builtin_nontemporal_load(static_cast<const u32x4*>(p));
  return uint4{v[0], v[1], v[2], v[3]};
}

__device__ __forceinline__ bf16x8 as_bf16x8(const uint4& v) {
  return __builtin_bit_cast(bf16x8, v);
}

__device__ __forceinline__ f32x4 mfma16(const uint4& a, const uint4& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

// Eight nibbles (two's complement q, element 8g + i in nibble i of w) as the
// A fragment of bf16 values 136 + q.
__device__ __forceinline__ uint4 int4_fragment(uint32_t w) {
  const uint32_t u = w ^ 0x88888888u;         // nibble i = q_i + 8
  const uint32_t lo = u & 0x0F0F0F0Fu;        // elements 0, 2, 4, 6 in bytes 0..3
  const uint32_t hi = (u >> 4) & 0x0F0F0F0Fu;  // elements 1, 3, 5, 7
  // interleave: t0 = [e0 e1 e2 e3], t1 = [e4 e5 e6 e7] (bytes)
  const uint32_t t0 = __builtin_amdgcn_perm(hi, lo, 0x05010400u);
  const uint32_t t1 = __builtin_amdgcn_perm(hi, lo, 0x07030602u);
  // each element byte under the bf16 high byte 0x43 (128 + byte)
  const uint32_t c43 = 0x43434343u;
  return uint4{__builtin_amdgcn_perm(c43, t0, 0x04010400u), __builtin_amdgcn_perm(c43, t0, 0x04030402u),
               __builtin_amdgcn_perm(c43, t1, 0x04010400u), __builtin_amdgcn_perm(c43, t1, 0x04030402u)};
}

// Eight int8 codes (element i in byte i of w) as the A fragment of bf16
// values q (|q| <= 127 is exact in bf16): sign-extend, convert, keep the
// high half.
__device__ __forceinline__ uint4 int8_fragment(const uint2& w) {
  uint32_t o[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t word = j < 2 ? w.x : w.y;
    const int sh = 16 * (j & 1);
    const float lo = (float)(int8_t)((word >> sh) & 0xFFu);
    const float hi = (float)(int8_t)((word >> (sh + 8)) & 0xFFu);
    o[j] = (__float_as_uint(lo) >> 16) | (__float_as_uint(hi) & 0xFFFF0000u);
  }
  return uint4{o[0], o[1], o[2], o[3]};
}

struct MfmaArgs {
  const void* A;           // bf16 rows [R x d], INT4 rows in the MFMA layout, or int8 rows [R x d]
  const uint16_t* sigT;    // INT4 / INT8: fp16 scales [G x ldsig], group-major
  int64_t ldsig;           // INT4 / INT8: rows per scale row (R rounded up to 128)
  int64_t a_row_bytes;     // INT4: bytes per re-laid row (64 per 4 groups)
  int64_t R;
  int d;
  const uint16_t* H;  // [B x d] bf16
  int B;
  float* out;  // [B x ld_out] scores / logits, or null
  int64_t ld_out;
  int token_sample;  // EPI
  float tprime;
  uint64_t seed;
  Part* parts;  // EPI: [B x gridDim.x]
  // EPI, speculative verification: with bits set, a token whose cluster
  // t2c[t] is among query q's probes (bit of bits[q W + k / 32]) gets key
  // -inf, any other z / T' + G(seed, q, t, stage 3); the LSE is unchanged
  const int32_t* t2c;
  const uint32_t* bits;
  int W;
  // optional row map (stage 2 over a probe list shared by the batch): logical
  // row r is row S[r / bsz] * bsz + r % bsz of A (the cluster-contiguous E),
  // its token C2T of that row; out_ids[q * ld_out + r] receives the token
  const int32_t* rows_map;
  int bsz;
  const int32_t* c2t;
  int32_t* out_ids;
  KeyXform key;  // stage 1 (not EPI): scores or selection keys into out
  // rows from a fragment-order copy (FRAG): row r's tile r / 16 at
  // Afrag + (r / 16) ns 64.  Stage 1: the centroids.  The dense passes (EPI):
  // the fragment-order E, row r is slot r of the clustering, its token c2t[r]
  // and its cluster r / bsz
  const uint4* Afrag;
  int ns;
};

constexpr int kHRow = 128 + 8;  // LDS row of a staged h block (bf16), padded

template <int NT, int MT, int QB, bool EPI, bool FRAG = false>
__global__ __launch_bounds__(256) void k_mfma_gemm(MfmaArgs a) {
  static_assert(!FRAG || QB == 0, "fragment-order rows are bf16");
  constexpr int QW = 16 * NT;  // queries per workgroup
  __shared__ __attribute__((aligned(16))) uint16_t sH[2][QW * kHRow];
  __shared__ Part sh[EPI ? 4 : 1][EPI ? QW : 1];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, col = lane & 15;
  const int64_t rbase = (int64_t)blockIdx.x * (64 * MT) + wave * (16 * MT);
  const int q0 = blockIdx.y * QW;
  const int nkb = (a.d + 127) / 128;

  // the queries' block kb of h -> registers (NT 16-byte chunks per thread)
  uint4 hreg[NT];
  auto load_h = [&](int kb) {
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      const int idx = tid + 256 * i, row = idx >> 4, c16 = idx & 15;
      const int k = 128 * kb + 8 * c16;
      const int q = min(q0 + row, a.B - 1);
      hreg[i] = k < a.d ? *reinterpret_cast<const uint4*>(a.H + (int64_t)q * a.d + k)
                        : uint4{0u, 0u, 0u, 0u};
    }
  };
  auto store_h = [&](int buf) {
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      const int idx = tid + 256 * i, row = idx >> 4, c16 = idx & 15;
      *reinterpret_cast<uint4*>(&sH[buf][row * kHRow + 8 * c16]) = hreg[i];
    }
  };

  f32x4 acc[MT][NT];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int n = 0; n < NT; ++n) acc[m][n] = f32x4{0.f, 0.f, 0.f, 0.f};

  // this lane's rows (clamped for loads; results past R are dropped), as
  // rows of A (through the row map when there is one)
  auto phys = [&](int64_t r) -> int64_t {
    return a.rows_map ? (int64_t)a.rows_map[r / a.bsz] * a.bsz + r % a.bsz : r;
  };
  int64_t ra[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) ra[m] = phys(min(rbase + 16 * m + col, a.R - 1));

  if constexpr (QB == 0) {
    const uint16_t* A = static_cast<const uint16_t*>(a.A);
    uint4 av[2][MT][4];
    auto load_a = [&](int kb, uint4 (&dst)[MT][4]) {
#pragma unroll
      for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          if constexpr (FRAG) {  // one contiguous 1 KB per instruction
            const int64_t tile = min((rbase + 16 * m) / 16, (a.R + 15) / 16 - 1);
            dst[m][s] = 4 * kb + s < a.ns ? ld_stream(a.Afrag + (tile * a.ns + 4 * kb + s) * 64 + lane)
                                          : uint4{0u, 0u, 0u, 0u};
          } else {
            const int k = 128 * kb + 32 * s + 8 * g;
            dst[m][s] = k < a.d ? *reinterpret_cast<const uint4*>(A + ra[m] * a.d + k)
                                : uint4{0u, 0u, 0u, 0u};
          }
        }
    };
    auto compute = [&](int buf, const uint4 (&cur)[MT][4]) {
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        uint4 bfr[NT];
#pragma unroll
        for (int n = 0; n < NT; ++n)
          bfr[n] = *reinterpret_cast<const uint4*>(&sH[buf][(16 * n + col) * kHRow + 32 * s + 8 * g]);
#pragma unroll
        for (int m = 0; m < MT; ++m)
#pragma unroll
          for (int n = 0; n < NT; ++n) acc[m][n] = mfma16(cur[m][s], bfr[n], acc[m][n]);
      }
    };
    load_h(0);
    load_a(0, av[0]);
    store_h(0);
    __syncthreads();
    for (int kb = 0; kb < nkb; kb += 2) {
      if (kb + 1 < nkb) {
        load_h(kb + 1);
        load_a(kb + 1, av[1]);
      }
      compute(0, av[0]);
      if (kb + 1 < nkb) store_h(1);
      __syncthreads();
      if (kb + 1 < nkb) {
        if (kb + 2 < nkb) {
          load_h(kb + 2);
          load_a(kb + 2, av[0]);
        }
        compute(1, av[1]);
        if (kb + 2 < nkb) store_h(0);
        __syncthreads();
      }
    }
  } else if constexpr (QB == 4) {
    const uint8_t* A = static_cast<const uint8_t*>(a.A);
    const int G = a.d / 32;
    const uint4 neg136 = uint4{0xC308C308u, 0xC308C308u, 0xC308C308u, 0xC308C308u};
    struct Blk {
      uint4 w[MT];
      uint2 sg[MT][4];
    };
    auto load_a = [&](int kb, Blk& x) {
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        const int64_t tile = min((rbase + 16 * m) / 16, (a.R + 15) / 16 - 1);
        x.w[m] = *reinterpret_cast<const uint4*>(A + ((tile * (a.a_row_bytes / 64) + kb) * 64 + lane) * 16);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const int grp = min(4 * kb + s, G - 1);
          x.sg[m][s] = *reinterpret_cast<const uint2*>(a.sigT + (int64_t)grp * a.ldsig + rbase +
                                                       16 * m + 4 * g);
        }
      }
    };
    auto compute = [&](int kb, int buf, const Blk& x) {
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        if (4 * kb + s >= G) break;
        uint4 bfr[NT];
#pragma unroll
        for (int n = 0; n < NT; ++n)
          bfr[n] = *reinterpret_cast<const uint4*>(&sH[buf][(16 * n + col) * kHRow + 32 * s + 8 * g]);
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          const uint32_t wv[4] = {x.w[m].x, x.w[m].y, x.w[m].z, x.w[m].w};
          const uint4 af = int4_fragment(wv[s]);
          const float sig[4] = {
              __half2float(__ushort_as_half((uint16_t)(x.sg[m][s].x & 0xFFFFu))),
              __half2float(__ushort_as_half((uint16_t)(x.sg[m][s].x >> 16))),
              __half2float(__ushort_as_half((uint16_t)(x.sg[m][s].y & 0xFFFFu))),
              __half2float(__ushort_as_half((uint16_t)(x.sg[m][s].y >> 16)))};
#pragma unroll
          for (int n = 0; n < NT; ++n) {
            f32x4 part = mfma16(af, bfr[n], f32x4{0.f, 0.f, 0.f, 0.f});
            part = mfma16(neg136, bfr[n], part);
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[m][n][i] = fmaf(sig[i], part[i], acc[m][n][i]);
          }
        }
      }
    };
    Blk x0, x1;
    load_h(0);
    load_a(0, x0);
    store_h(0);
    __syncthreads();
    for (int kb = 0; kb < nkb; kb += 2) {
      if (kb + 1 < nkb) {
        load_h(kb + 1);
        load_a(kb + 1, x1);
      }
      compute(kb, 0, x0);
      if (kb + 1 < nkb) store_h(1);
      __syncthreads();
      if (kb + 1 < nkb) {
        if (kb + 2 < nkb) {
          load_h(kb + 2);
          load_a(kb + 2, x0);
        }
        compute(kb + 1, 1, x1);
        if (kb + 2 < nkb) store_h(0);
        __syncthreads();
      }
    }
  } else {
    // INT8 rows, row-major (d bytes per row): MFMA step s of block kb is
    // group 4 kb + s; lane group g takes its elements 8 g .. + 7 (8 bytes),
    // widened exactly to bf16; the group's fp16 scales then scale the tile
    // into the running score with one FMA per element
    static_assert(QB == 8, "QB is 0, 4 or 8");
    const uint8_t* A = static_cast<const uint8_t*>(a.A);
    const int G = a.d / 32;
    struct Blk {
      uint2 w[MT][4];
      uint2 sg[MT][4];
    };
    auto load_a = [&](int kb, Blk& x) {
#pragma unroll
      for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const int grp = min(4 * kb + s, G - 1);
          x.w[m][s] = *reinterpret_cast<const uint2*>(A + ra[m] * a.d + 32 * grp + 8 * g);
          x.sg[m][s] = *reinterpret_cast<const uint2*>(a.sigT + (int64_t)grp * a.ldsig + rbase +
                                                       16 * m + 4 * g);
        }
    };
    auto compute = [&](int kb, int buf, const Blk& x) {
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        if (4 * kb + s >= G) break;
        uint4 bfr[NT];
#pragma unroll
        for (int n = 0; n < NT; ++n)
          bfr[n] = *reinterpret_cast<const uint4*>(&sH[buf][(16 * n + col) * kHRow + 32 * s + 8 * g]);
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          const uint4 af = int8_fragment(x.w[m][s]);
          const float sig[4] = {
              __half2float(__ushort_as_half((uint16_t)(x.sg[m][s].x & 0xFFFFu))),
              __half2float(__ushort_as_half((uint16_t)(x.sg[m][s].x >> 16))),
              __half2float(__ushort_as_half((uint16_t)(x.sg[m][s].y & 0xFFFFu))),
              __half2float(__ushort_as_half((uint16_t)(x.sg[m][s].y >> 16)))};
#pragma unroll
          for (int n = 0; n < NT; ++n) {
            const f32x4 part = mfma16(af, bfr[n], f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[m][n][i] = fmaf(sig[i], part[i], acc[m][n][i]);
          }
        }
      }
    };
    Blk x0, x1;
    load_h(0);
    load_a(0, x0);
    store_h(0);
    __syncthreads();
    for (int kb = 0; kb < nkb; kb += 2) {
      if (kb + 1 < nkb) {
        load_h(kb + 1);
        load_a(kb + 1, x1);
      }
      compute(kb, 0, x0);
      if (kb + 1 < nkb) store_h(1);
      __syncthreads();
      if (kb + 1 < nkb) {
        if (kb + 2 < nkb) {
          load_h(kb + 2);
          load_a(kb + 2, x0);
        }
        compute(kb + 1, 1, x1);
        if (kb + 2 < nkb) store_h(0);
        __syncthreads();
      }
    }
  }

  // lane holds rows rbase + 16 m + 4 g + i (i < 4) of queries q0 + 16 n + col
  if (!EPI) {
    if (a.out) {
#pragma unroll
      for (int n = 0; n < NT; ++n) {
        const int q = q0 + 16 * n + col;
        if (q >= a.B) continue;
#pragma unroll
        for (int m = 0; m < MT; ++m)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int64_t r = rbase + 16 * m + 4 * g + i;
            if (r < a.R)
              a.out[(int64_t)q * a.ld_out + r] = stage1_value(
                  acc[m][n][i], a.key.sample, a.key.temperature, a.key.seed, (uint32_t)q, (uint32_t)r);
          }
      }
    }
    return;
  }
#pragma unroll
  for (int n = 0; n < NT; ++n) {
    const int q = q0 + 16 * n + col;
    Part p = part_empty();
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t r = rbase + 16 * m + 4 * g + i;
        if (r < a.R && q < a.B) {
          const int32_t tok = FRAG ? a.c2t[r] : a.rows_map ? a.c2t[phys(r)] : (int32_t)r;
          // the dense logits at the token's position (slots under FRAG)
          if (a.out) a.out[(int64_t)q * a.ld_out + (FRAG ? (int64_t)tok : r)] = acc[m][n][i];
          if (a.out_ids) a.out_ids[(int64_t)q * a.ld_out + r] = tok;
          Part pt = part_of(acc[m][n][i], tok, a.token_sample, a.tprime, a.seed, (uint32_t)q);
          if (a.bits) {
            const int k = FRAG ? (int)(r / a.bsz) : a.t2c[r];
            const bool probed = (a.bits[(int64_t)q * a.W + (k >> 5)] >> (k & 31)) & 1u;
            pt.key = probed ? -INFINITY
                            : acc[m][n][i] / a.tprime + gumbel_at(a.seed, (uint32_t)q, (uint32_t)tok, 3u);
          }
          p = part_merge(p, pt);
        }
      }
    // the four lane groups hold the same query: fold them (fixed order)
#pragma unroll
    for (int msk = 16; msk <= 32; msk *= 2) {
      const Part o{__shfl_xor(p.key, msk), __shfl_xor(p.z, msk), __shfl_xor(p.m, msk),
                   __shfl_xor(p.s, msk), __shfl_xor(p.id, msk)};
      p = (lane & msk) ? part_merge(o, p) : part_merge(p, o);
    }
    if (g == 0) sh[wave][16 * n + col] = p;
  }
  __syncthreads();
  if (tid < QW) {
    const int q = q0 + tid;
    Part r = sh[0][tid];
#pragma unroll
    for (int w = 1; w < 4; ++w) r = part_merge(r, sh[w][tid]);
    if (q < a.B) a.parts[(int64_t)q * gridDim.x + blockIdx.x] = r;
  }
}

// ======================================================================
// Stage 1 split over d, one 16-query tile per workgroup row (grid.y).  With
// one query tile per workgroup the GEMM above has one workgroup per 64 rows
// and tile (126 per tile at the Llama-3.2-1B shape's 8016 centroids), each
// walking all of d; its time is the chain of d / 128 dependent block steps.
// Here the four waves of a workgroup take the same 16 rows and consecutive
// quarters of d, so there are four times the workgroups and a quarter of the
// chain per wave.  Each
// lane loads its queries' h fragments itself (the [B x d] queries are a few
// KB and stay in cache), so the waves never synchronise until the end, where
// waves 1..3 hand their tiles to wave 0 through LDS and it adds them in wave
// order.  Rows and scale layout as in k_mfma_gemm (MT = 1, no row map).
// ======================================================================
template <int QB, bool EPI, bool FRAG = false>
__global__ __launch_bounds__(256) void k_mfma_stage1_splitd(MfmaArgs a) {
  static_assert(!FRAG || QB == 0, "fragment-order rows are bf16");
  __shared__ f32x4 red[3][64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, col = lane & 15;
  const int64_t rbase = (int64_t)blockIdx.x * 16;
  const int q0 = 16 * blockIdx.y;
  const int nkb = (a.d + 127) / 128;
  const int kb0 = wave * nkb / 4, kb1 = (wave + 1) * nkb / 4;
  const uint16_t* Hq = a.H + (int64_t)min(q0 + col, a.B - 1) * a.d;
  const int64_t ra = min(rbase + col, a.R - 1);
  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
  // the queries' fragments of block kb: step s holds elements 128 kb + 32 s + 8 g .. + 7
  auto load_h = [&](int kb, uint4 (&hb)[4]) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int k = 128 * kb + 32 * s + 8 * g;
      hb[s] = k < a.d ? *reinterpret_cast<const uint4*>(Hq + k) : uint4{0u, 0u, 0u, 0u};
    }
  };
  if constexpr (QB == 0) {
    const uint16_t* A = static_cast<const uint16_t*>(a.A);
    struct Blk {
      uint4 v[4], hb[4];
    };
    auto load = [&](int kb, Blk& x) {
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        if constexpr (FRAG) {  // one contiguous 1 KB per instruction
          const int64_t tile = rbase / 16;  // the grid covers ceil(R / 16) tiles
          x.v[s] = 4 * kb + s < a.ns ? ld_stream(a.Afrag + (tile * a.ns + 4 * kb + s) * 64 + lane)
                                     : uint4{0u, 0u, 0u, 0u};
        } else {
          const int k = 128 * kb + 32 * s + 8 * g;
          x.v[s] = k < a.d ? *reinterpret_cast<const uint4*>(A + ra * a.d + k) : uint4{0u, 0u, 0u, 0u};
        }
      }
      load_h(kb, x.hb);
    };
    auto compute = [&](int, const Blk& x) {
#pragma unroll
      for (int s = 0; s < 4; ++s) acc = mfma16(x.v[s], x.hb[s], acc);
    };
    Blk b0, b1;
    if (kb0 < kb1) load(kb0, b0);
    for (int kb = kb0; kb < kb1; kb += 2) {
      if (kb + 1 < kb1) load(kb + 1, b1);
      compute(kb, b0);
      if (kb + 1 < kb1) {
        if (kb + 2 < kb1) load(kb + 2, b0);
        compute(kb + 1, b1);
      }
    }
  } else {
    const uint8_t* A = static_cast<const uint8_t*>(a.A);
    const int G = a.d / 32;
    const uint4 neg136 = uint4{0xC308C308u, 0xC308C308u, 0xC308C308u, 0xC308C308u};
    struct Blk {
      uint4 w4;       // INT4: lane group g's bytes of the block's four groups
      uint2 w8[4];    // INT8: lane group g's 8 bytes of each group
      uint2 sg[4];
      uint4 hb[4];
    };
    auto load = [&](int kb, Blk& x) {
      if constexpr (QB == 4)  // fragment order: the grid covers ceil(R / 16) tiles
        x.w4 = *reinterpret_cast<const uint4*>(A + ((rbase / 16 * (a.a_row_bytes / 64) + kb) * 64 + lane) * 16);
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int grp = min(4 * kb + s, G - 1);
        if constexpr (QB == 8)
          x.w8[s] = *reinterpret_cast<const uint2*>(A + ra * a.d + 32 * grp + 8 * g);
        x.sg[s] = *reinterpret_cast<const uint2*>(a.sigT + (int64_t)grp * a.ldsig + rbase + 4 * g);
      }
      load_h(kb, x.hb);
    };
    auto compute = [&](int kb, const Blk& x) {
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        if (4 * kb + s >= G) break;
        f32x4 part;
        if constexpr (QB == 4) {
          const uint32_t wv[4] = {x.w4.x, x.w4.y, x.w4.z, x.w4.w};
          part = mfma16(int4_fragment(wv[s]), x.hb[s], f32x4{0.f, 0.f, 0.f, 0.f});
          part = mfma16(neg136, x.hb[s], part);
        } else {
          part = mfma16(int8_fragment(x.w8[s]), x.hb[s], f32x4{0.f, 0.f, 0.f, 0.f});
        }
        const float sig[4] = {
            __half2float(__ushort_as_half((uint16_t)(x.sg[s].x & 0xFFFFu))),
            __half2float(__ushort_as_half((uint16_t)(x.sg[s].x >> 16))),
            __half2float(__ushort_as_half((uint16_t)(x.sg[s].y & 0xFFFFu))),
            __half2float(__ushort_as_half((uint16_t)(x.sg[s].y >> 16)))};
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] = fmaf(sig[i], part[i], acc[i]);
      }
    };
    Blk b0, b1;
    if (kb0 < kb1) load(kb0, b0);
    for (int kb = kb0; kb < kb1; kb += 2) {
      if (kb + 1 < kb1) load(kb + 1, b1);
      compute(kb, b0);
      if (kb + 1 < kb1) {
        if (kb + 2 < kb1) load(kb + 2, b0);
        compute(kb + 1, b1);
      }
    }
  }
  if (wave > 0) red[wave - 1][lane] = acc;
  __syncthreads();
  if (wave > 0) return;
#pragma unroll
  for (int w = 0; w < 3; ++w) {
    const f32x4 o = red[w][lane];
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] += o[i];
  }
  // lane holds rows rbase + 4 g + i of query q0 + col
  const int q = q0 + col;
  if constexpr (EPI) {
    // the dense head's epilogue (as in k_mfma_gemm, rows are tokens): one
    // partial per query and workgroup, the four lane groups folded in order
    Part p = part_empty();
    const bool qok = q < a.B;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t r = rbase + 4 * g + i;
      if (qok && r < a.R) {
        const int32_t tok = FRAG ? a.c2t[r] : (int32_t)r;  // slots under FRAG
        if (a.out) a.out[(int64_t)q * a.ld_out + tok] = acc[i];
        Part pt = part_of(acc[i], tok, a.token_sample, a.tprime, a.seed, (uint32_t)q);
        if (a.bits) {
          const int k = FRAG ? (int)(r / a.bsz) : a.t2c[r];
          const bool probed = (a.bits[(int64_t)q * a.W + (k >> 5)] >> (k & 31)) & 1u;
          pt.key = probed ? -INFINITY
                          : acc[i] / a.tprime + gumbel_at(a.seed, (uint32_t)q, (uint32_t)tok, 3u);
        }
        p = part_merge(p, pt);
      }
    }
#pragma unroll
    for (int msk = 16; msk <= 32; msk *= 2) {
      const Part o{__shfl_xor(p.key, msk), __shfl_xor(p.z, msk), __shfl_xor(p.m, msk),
                   __shfl_xor(p.s, msk), __shfl_xor(p.id, msk)};
      p = (lane & msk) ? part_merge(o, p) : part_merge(p, o);
    }
    if (g == 0 && qok) a.parts[(int64_t)q * gridDim.x + blockIdx.x] = p;
    return;
  }
  if (q >= a.B) return;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t r = rbase + 4 * g + i;
    if (r < a.R)
      a.out[(int64_t)q * a.ld_out + r] =
          stage1_value(acc[i], a.key.sample, a.key.temperature, a.key.seed, (uint32_t)q, (uint32_t)r);
  }
}

// ======================================================================
// Cluster-major stage 2 (explainer §1.2.1, §1.2.4; batch semantics: each
// query still takes only its own probes).  Workgroup x owns clusters
// [8x, 8x + 8).  For each of them the workgroup lists the queries whose
// probe bitset holds it (ballots over the bitset words, ascending query
// order).  The work items -- (cluster, tile of 16 of its rows, tile of 16 of
// its queries) -- are taken round-robin by the four waves; each computes its
// 16 x 16 logits with MFMA over d (the next 128-element block's loads in
// flight during the current block's products), so a cluster's rows are read
// once for all its queries and a much-probed cluster's query tiles run in
// parallel.  The rows come from the fragment-order copy of E (Ecm, below),
// so every row load is one contiguous 1 KB read.  The epilogue writes the
// optional outputs at the query's canonical position (probe rank from the
// bitset and its word prefix counts, then slot) and one partial per query,
// probe rank and row tile at parts[(q p + rank) nrt + rt], so that every
// query's partials are merged in ascending cluster order whichever
// workgroup ran first.
//
// Ecm, the fragment-order copy of the cluster-contiguous E (bf16 engines
// that take batches): row tile rt of cluster k is ns = ceil(d / 32) steps of
// 1 KB at tile index k nrt + rt; step s holds, for lane group g and row col,
// elements 32 s + 8 g .. + 7 of the cluster's row 16 rt + col at byte
// ((4 s + g) 16 + col) 16 -- the fragment lane 16 g + col of the MFMA takes
// -- and zeros past the cluster's rows and past d.  (Read from the
// row-major copy, an instruction touches 16 rows x 64 B; measured on the
// Qwen-3-4B shape's 778 MB, that order streams at 4.4 TB/s where 1 KB
// pieces stream at 6.0 and a plain read at 6.9.)
// ======================================================================
// Clusters per workgroup; divides 32 (one bitset word).  Small workgroups
// balance best: measured at 8 / 4 / 2 / 1 clusters, Qwen-3-4B INT4 B = 128
// 236.8 / 234.0 / 224.7 / 223.9 us per call, Llama INT4 B = 32
// 106.7 / 103.5 / 102.0 / 100.5 us.
constexpr int kCmClusters = 1;
static_assert(32 % kCmClusters == 0, "a workgroup's clusters share one bitset word");
constexpr int kCmMaxB = 256;    // queries the LDS lists hold

struct GatherCmArgs {
  const uint4* Ecm;    // fragment-order copy of E (above)
  const int32_t* c2t;
  int c, b, d;
  const uint16_t* H;  // [B x d]
  int B, p;
  const uint32_t* mbits;  // [W x B] probe bitset words
  const int32_t* mpre;    // [W x B] probes in earlier words
  int32_t* out_ids;       // [B x p b] or null
  float* out_logits;      // [B x p b] or null
  int token_sample;
  float tprime;
  uint64_t seed;
  Part* parts;  // [B x p nrt]
};

__global__ __launch_bounds__(256) void k_gather_cm(GatherCmArgs a) {
  __shared__ uint32_t s_word[kCmMaxB];
  __shared__ int s_pre[kCmMaxB];
  __shared__ short s_q[kCmClusters][kCmMaxB];
  __shared__ int s_n[kCmClusters];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, col = lane & 15;
  const int k0 = blockIdx.x * kCmClusters;
  const int w = k0 >> 5;  // the workgroup's clusters share one bitset word
  for (int q = threadIdx.x; q < a.B; q += 256) {
    s_word[q] = a.mbits[(int64_t)w * a.B + q];
    s_pre[q] = a.mpre[(int64_t)w * a.B + q];
  }
  __syncthreads();
  // the queries probing each of the workgroup's clusters, ascending
  for (int ci = wave; ci < kCmClusters; ci += 4) {
    const int k = k0 + ci;
    int n = 0;
    if (k < a.c) {
      const int bit = k & 31;
      for (int qb = 0; qb < a.B; qb += 64) {
        const int q = qb + lane;
        const bool in = q < a.B && ((s_word[q] >> bit) & 1u);
        const unsigned long long m = __ballot(in);
        if (in)
          s_q[ci][n + __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u))] = (short)q;
        n += __popcll(m);
      }
    }
    if (lane == 0) s_n[ci] = n;
  }
  __syncthreads();
  // work items (cluster, row tile, query tile), in that order, taken round-
  // robin by the four waves: a cluster probed by many queries spreads its
  // query tiles over the waves
  const int nrt = (a.b + 15) / 16, ns = (a.d + 31) / 32;
  int total = 0;
#pragma unroll
  for (int ci = 0; ci < kCmClusters; ++ci) total += nrt * ((s_n[ci] + 15) / 16);
  const int64_t ldo = (int64_t)a.p * a.b;
  for (int it = wave; it < total; it += 4) {
    int ci = 0, rem = it;
    for (; ci < kCmClusters; ++ci) {
      const int cnt = nrt * ((s_n[ci] + 15) / 16);
      if (rem < cnt) break;
      rem -= cnt;
    }
    const int n = s_n[ci];
    const int nqt = (n + 15) / 16;
    const int rt = rem / nqt, qt = rem % nqt;
    const int k = k0 + ci;
    const int bit = k & 31;
    // step s of the tile: At[64 s], the lane's fragment
    const uint4* At = a.Ecm + ((int64_t)k * nrt + rt) * ns * 64 + lane;
    // the tile's token ids, loaded ahead of the products
    int32_t tok[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) tok[i] = a.c2t[(int64_t)k * a.b + min(16 * rt + 4 * g + i, a.b - 1)];
    const int qi = 16 * qt + col;
    const int q = s_q[ci][min(qi, n - 1)];
    const uint16_t* Hr = a.H + (int64_t)q * a.d;
    const int nblk = a.d / 128;
    // The tile's products.  A tile read by one query tile only is streamed
    // with the non-temporal hint; a tile that several query tiles read keeps
    // ordinary loads, so that the later reads find it in cache (measured both
    // ways: the hint alone took Llama INT4 B = 64 from 135 to 119 us and the
    // Qwen B = 128 call from 238 to 245 us).
    auto products = [&](auto stream) -> f32x4 {
      constexpr bool kStream = decltype(stream)::value;
      auto ld_a = [&](int st) -> uint4 {
        if constexpr (kStream) return ld_stream(At + 64 * st);
        else return At[64 * st];
      };
      f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
      // ping-pong: the next 128-element block (four steps) is in flight
      // during the current block's products
      uint4 a0[4], b0[4], a1[4], b1[4];
      auto ld = [&](int blk, uint4 (&av)[4], uint4 (&bv)[4]) {
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          av[s] = ld_a(4 * blk + s);
          bv[s] = *reinterpret_cast<const uint4*>(Hr + 128 * blk + 32 * s + 8 * g);
        }
      };
      if (nblk > 0) ld(0, a0, b0);
      for (int blk = 0; blk < nblk; blk += 2) {
        if (blk + 1 < nblk) ld(blk + 1, a1, b1);
#pragma unroll
        for (int s = 0; s < 4; ++s) acc = mfma16(a0[s], b0[s], acc);
        if (blk + 1 < nblk) {
          if (blk + 2 < nblk) ld(blk + 2, a0, b0);
#pragma unroll
          for (int s = 0; s < 4; ++s) acc = mfma16(a1[s], b1[s], acc);
        }
      }
      for (int st = 4 * nblk; st < ns; ++st) {  // d % 128 != 0: the last steps (Ecm is zero past d)
        const int kk = 32 * st + 8 * g;
        const uint4 bv = kk < a.d ? *reinterpret_cast<const uint4*>(Hr + kk) : uint4{0u, 0u, 0u, 0u};
        acc = mfma16(ld_a(st), bv, acc);
      }
      return acc;
    };
    const f32x4 acc = nqt == 1 ? products(std::true_type{}) : products(std::false_type{});
    // lane: slots j = 16 rt + 4 g + i of cluster k for query q
    const bool qok = qi < n;
    const int pos = qok ? s_pre[q] + __popc(s_word[q] & ((1u << bit) - 1u)) : 0;
    Part pt = part_empty();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int j = 16 * rt + 4 * g + i;
      if (qok && j < a.b) {
        const int64_t o = (int64_t)q * ldo + (int64_t)pos * a.b + j;
        if (a.out_logits) a.out_logits[o] = acc[i];
        if (a.out_ids) a.out_ids[o] = tok[i];
        pt = part_merge(pt, part_of(acc[i], tok[i], a.token_sample, a.tprime, a.seed, (uint32_t)q));
      }
    }
#pragma unroll
    for (int m = 16; m <= 32; m *= 2) {
      const Part o{__shfl_xor(pt.key, m), __shfl_xor(pt.z, m), __shfl_xor(pt.m, m),
                   __shfl_xor(pt.s, m), __shfl_xor(pt.id, m)};
      pt = (lane & m) ? part_merge(o, pt) : part_merge(pt, o);
    }
    if (g == 0 && qok) a.parts[((int64_t)q * a.p + pos) * nrt + rt] = pt;
  }
}

// The fragment-order copy (layout above) of c clusters of b contiguous rows
// each: one thread per 16-byte fragment.  With c = 1 and b = the row count it
// is a plain matrix's tiles of 16 consecutive rows (the centroids).
__global__ __launch_bounds__(256) void k_fragment_order(const uint16_t* __restrict__ Ec, int64_t c,
                                                        int b, int d, int nrt, int ns,
                                                        uint4* __restrict__ out) {
  const int64_t o = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (o >= c * nrt * ns * 64) return;
  const int lane = (int)(o & 63);
  const int64_t step = o >> 6;
  const int s = (int)(step % ns);
  const int64_t tile = step / ns;
  const int64_t k = tile / nrt;
  const int rt = (int)(tile % nrt);
  const int r = 16 * rt + (lane & 15), e = 32 * s + 8 * (lane >> 4);
  out[o] = r < b && e < d ? *reinterpret_cast<const uint4*>(Ec + (k * b + r) * d + e)
                          : uint4{0u, 0u, 0u, 0u};
}

// Re-lay INT4 rows for the MFMA tiles, in fragment order: tiles of 16 rows,
// and in tile t, block kb (four groups, 128 elements) is 1 KB in which lane
// 16 g + col's 16 bytes are lane group g's four bytes of each of the four
// groups (elements 8g .. 8g+7) of row 16 t + col -- so one load instruction
// reads 1 KB in one piece.  Zero codes past the row's groups and past c.
// One thread per 16-byte output chunk.
__global__ __launch_bounds__(256) void k_relayout_int4(const uint8_t* __restrict__ q, int64_t c,
                                                       int G, uint8_t* __restrict__ out,
                                                       int64_t row_bytes) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;  // output chunk
  const int64_t nkb = row_bytes / 64;
  if (i >= (c + 15) / 16 * 16 * (row_bytes / 16)) return;
  const int lane = (int)(i & 63), g = lane >> 4;
  const int64_t kb = (i >> 6) % nkb, t = (i >> 6) / nkb;
  const int64_t r = 16 * t + (lane & 15);
  uint32_t w[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int64_t grp = 4 * kb + s;
    w[s] = r < c && grp < G ? *reinterpret_cast<const uint32_t*>(q + r * (G * 16) + grp * 16 + 4 * g) : 0u;
  }
  *reinterpret_cast<uint4*>(out + 16 * i) = uint4{w[0], w[1], w[2], w[3]};
}

// Scales group-major: sigT[grp][r] = sig[r][grp] (rows past c are 0).
__global__ __launch_bounds__(256) void k_transpose_sig(const uint16_t* __restrict__ sig, int64_t c,
                                                       int G, int64_t ld, uint16_t* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)G * ld) return;
  const int64_t grp = i / ld, r = i % ld;
  out[i] = r < c ? sig[r * G + grp] : (uint16_t)0;
}

// ----------------------------------------------------------------- host ---

int64_t mfma_int4_row_bytes(int d) { return (int64_t)((d / 32 + 3) / 4) * 64; }
// Rows per group of the group-major scales: every row a workgroup of the
// GEMM covers (64 MT <= 128 rows per workgroup), zero past c, so the scale
// loads of the last workgroup stay inside the table.
int64_t mfma_sig_ld(int64_t c) { return (c + 127) / 128 * 128; }

hipError_t launch_mfma_relayout(const KernelCtx& k, uint8_t* cq_mfma, uint16_t* sigT) {
  const int G = k.d / 32;
  if (k.qbits == 4) {  // INT8 rows are read as stored
    const int64_t rb = mfma_int4_row_bytes(k.d);
    const int64_t chunks = (k.c + 15) / 16 * 16 * (rb / 16);
    hipLaunchKernelGGL(k_relayout_int4, dim3((unsigned)((chunks + 255) / 256)), dim3(256), 0,
                       k.stream, k.cq, k.c, G, cq_mfma, rb);
    const hipError_t r = hipGetLastError();
    if (r != hipSuccess) return r;
  }
  const int64_t ld = mfma_sig_ld(k.c);
  hipLaunchKernelGGL(k_transpose_sig, dim3((unsigned)((G * ld + 255) / 256)), dim3(256), 0,
                     k.stream, k.csig, k.c, G, ld, sigT);
  return hipGetLastError();
}

// Tile shape: all query tiles in one workgroup (up to 8: the rows are read
// once), two row tiles per wave.  One row tile when that leaves fewer than 4
// workgroups per CU, then fewer query tiles per workgroup while there are
// fewer than 2 per CU.  Against thresholds of 2 and 1 this gives 37 us
// instead of 43 us for the INT4 stage 1 at 128 queries of the Qwen-3-4B
// shape and 149 us instead of 163 us for the dense head at 64 queries of the
// Llama-3.2-1B shape; 4 and 8 workgroups per CU gain no more.  With 8 query
// tiles a wave always keeps one row tile: two row tiles' accumulators and
// loads take more than half the register file (one wave per SIMD), and the
// dense head at 128 queries of the Qwen-3-4B shape took 511 us per call
// against 384 us, although every workgroup now stages h for half as many
// rows.
struct GemmShape {
  int nt, mt;
};
static GemmShape gemm_shape(int64_t R, int B, int cus) {
  const int tiles = (B + 15) / 16;
  GemmShape s{std::min(8, tiles) <= 1 ? 1 : std::min(8, tiles) <= 2 ? 2 : std::min(8, tiles) <= 4 ? 4 : 8, 2};
  auto wgs = [&](const GemmShape& x) {
    return ((R + 64 * x.mt - 1) / (64 * x.mt)) * ((tiles + x.nt - 1) / x.nt);
  };
  if (s.nt == 8 || wgs(s) < 4 * (int64_t)cus) s.mt = 1;
  while (s.nt > 1 && wgs(s) < 2 * (int64_t)cus) s.nt /= 2;
  return s;
}

template <int NT, int MT, int QB, bool EPI, bool FRAG>
static hipError_t gemm_go(const MfmaArgs& a, hipStream_t st, int64_t* nblocks) {
  const dim3 grid((unsigned)((a.R + 64 * MT - 1) / (64 * MT)),
                  (unsigned)((a.B + 16 * NT - 1) / (16 * NT)));
  if (nblocks) *nblocks = grid.x;
  hipLaunchKernelGGL((k_mfma_gemm<NT, MT, QB, EPI, FRAG>), grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

template <int MT, int QB, bool EPI, bool FRAG>
static hipError_t gemm_nt(const MfmaArgs& a, int nt, hipStream_t st, int64_t* nblocks) {
  switch (nt) {
    case 1: return gemm_go<1, MT, QB, EPI, FRAG>(a, st, nblocks);
    case 2: return gemm_go<2, MT, QB, EPI, FRAG>(a, st, nblocks);
    case 4: return gemm_go<4, MT, QB, EPI, FRAG>(a, st, nblocks);
    default: return gemm_go<8, MT, QB, EPI, FRAG>(a, st, nblocks);
  }
}

template <int QB, bool EPI, bool FRAG = false>
static hipError_t mfma_dispatch(const MfmaArgs& a, int cus, hipStream_t st, int64_t* nblocks) {
  const GemmShape s = gemm_shape(a.R, a.B, cus);
  return s.mt == 2 ? gemm_nt<2, QB, EPI, FRAG>(a, s.nt, st, nblocks)
                   : gemm_nt<1, QB, EPI, FRAG>(a, s.nt, st, nblocks);
}

int64_t mfma_blocks(int64_t R) { return (R + 63) / 64; }
int64_t splitd_blocks(int64_t R) { return (R + 15) / 16; }

// Stage 1 split over d up to 32 queries, where the GEMM's shape rule finds
// too few workgroups for more than one query tile per workgroup.  Measured at
// the Llama-3.2-1B shape (INT4 / bf16 stage 1): B = 8 10.4 / 11.6 us against
// 21.4 / 23.2 us, B = 32 18.0 / 20.9 us against 22.3 / 24.3 us; at B = 64 the
// GEMM is faster (22.8 / 30.8 us against 28.3 / 34.8 us), its rows being read
// once per workgroup for more queries.
template <int QB, bool FRAG = false>
static hipError_t score_mfma_go(const MfmaArgs& a, int cus, hipStream_t st) {
  const GemmShape s = gemm_shape(a.R, a.B, cus);
  const bool splitd = a.B <= 32 && s.nt == 1 && s.mt == 1;
  if (splitd) {
    const dim3 grid((unsigned)((a.R + 15) / 16), (unsigned)((a.B + 15) / 16));
    hipLaunchKernelGGL((k_mfma_stage1_splitd<QB, false, FRAG>), grid, dim3(256), 0, st, a);
    return hipGetLastError();
  }
  return mfma_dispatch<QB, false, FRAG>(a, cus, st, nullptr);
}

hipError_t launch_score_mfma(const KernelCtx& k, int cus, const void* h, int B, float* out,
                             const KeyXform& kx) {
  MfmaArgs a{};
  a.R = k.c; a.d = k.d; a.H = static_cast<const uint16_t*>(h); a.B = B;
  a.out = out; a.ld_out = k.c; a.key = kx;
  if (k.qbits == 4) {
    a.A = k.cq_mfma; a.sigT = k.sig_mfma; a.ldsig = mfma_sig_ld(k.c);
    a.a_row_bytes = mfma_int4_row_bytes(k.d);
    return score_mfma_go<4>(a, cus, k.stream);
  }
  if (k.qbits == 8) {
    a.A = k.cq; a.sigT = k.sig_mfma; a.ldsig = mfma_sig_ld(k.c);
    return score_mfma_go<8>(a, cus, k.stream);
  }
  a.A = k.C;
  if (k.Cm) {  // the centroids' fragment-order copy: one contiguous 1 KB per load
    a.Afrag = static_cast<const uint4*>(k.Cm);
    a.ns = (k.d + 31) / 32;
    return score_mfma_go<0, true>(a, cus, k.stream);
  }
  return score_mfma_go<0>(a, cus, k.stream);
}

// Cluster-major pays off when clusters are shared: the expected number of
// queries per probed cluster, B p / (c (1 - (1 - p/c)^B)), is at least 2.
int gather_cm_max_batch() { return kCmMaxB; }
bool gather_cm_fits(int B, int64_t p, int64_t c) {
  if (B < 2 || B > kCmMaxB) return false;
  const double f = (double)p / (double)c;
  const double u = (double)c * (1.0 - std::pow(1.0 - f, (double)B));
  // the batch reads each probed cluster for 1.2 queries or more on average
  // (measured against the query-major launch: Llama INT4 B = 16 96.8 ->
  // 78.6 us, Gemma B = 16 75.7 -> 72.1 us, Llama INT4 B = 8 60.3 -> 59.8 us)
  return (double)B * (double)p >= 1.2 * u;
}

int64_t fragment_order_bytes(int64_t c, int64_t b, int d) {
  return c * ((b + 15) / 16) * ((d + 31) / 32) * 1024;
}

hipError_t launch_fragment_order(const void* rows, int64_t c, int64_t b, int d, void* out,
                                 hipStream_t st) {
  const int nrt = (int)((b + 15) / 16), ns = (d + 31) / 32;
  const int64_t n = c * nrt * ns * 64;
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_fragment_order, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st,
                     static_cast<const uint16_t*>(rows), c, (int)b, d, nrt, ns,
                     static_cast<uint4*>(out));
  return hipGetLastError();
}

hipError_t launch_gather_cm(const KernelCtx& k, int cus, const void* h, int B, int p,
                            const uint32_t* mbits,
                            const int32_t* mpre, int token_sample, float tprime, uint64_t seed,
                            int32_t* out_ids, float* out_logits, Part* parts, int64_t* nparts) {
  (void)cus;
  if (!k.Ecm || B < 1 || B > kCmMaxB || p < 1) return hipErrorInvalidValue;
  GatherCmArgs a{};
  a.Ecm = static_cast<const uint4*>(k.Ecm); a.c2t = k.c2t;
  a.c = (int)k.c; a.b = (int)k.b; a.d = k.d;
  a.H = static_cast<const uint16_t*>(h); a.B = B; a.p = p;
  a.mbits = mbits; a.mpre = mpre; a.out_ids = out_ids; a.out_logits = out_logits;
  a.token_sample = token_sample; a.tprime = tprime; a.seed = seed; a.parts = parts;
  *nparts = (int64_t)p * ((k.b + 15) / 16);
  const int64_t blocks = (k.c + kCmClusters - 1) / kCmClusters;
  if (blocks <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_gather_cm, dim3((unsigned)blocks), dim3(256), 0, k.stream, a);
  return hipGetLastError();
}

// The dense head's passes over all of E (the dense head itself and the
// verification's): split over d for up to kDenseSplitdMaxB queries, the GEMM
// beyond.  Every 16-row workgroup of the split reads its queries' h, so the
// cache traffic grows with B: measured at the Llama-3.2-1B shape, B = 2 takes
// 101 us against the GEMM's 116 us, but B = 8 122 us against 118 us.
constexpr int kDenseSplitdMaxB = 4;
template <bool FRAG>
static hipError_t dense_mfma_go(const MfmaArgs& a, int cus, hipStream_t st, int64_t* nparts) {
  if (a.B <= kDenseSplitdMaxB) {
    const dim3 grid((unsigned)splitd_blocks(a.R), 1);
    *nparts = grid.x;
    hipLaunchKernelGGL((k_mfma_stage1_splitd<0, true, FRAG>), grid, dim3(256), 0, st, a);
    return hipGetLastError();
  }
  return mfma_dispatch<0, true, FRAG>(a, cus, st, nparts);
}

// The dense passes read the fragment-order copy of E when the engine keeps
// one and its 16-row tiles are consecutive slots (b a multiple of 16).
static hipError_t dense_rows_go(const KernelCtx& k, MfmaArgs& a, int cus, int64_t* nparts) {
  if (k.Ecm && k.b % 16 == 0) {
    a.Afrag = static_cast<const uint4*>(k.Ecm);
    a.ns = (k.d + 31) / 32;
    a.c2t = k.c2t;
    a.bsz = (int)k.b;
    return dense_mfma_go<true>(a, cus, k.stream, nparts);
  }
  return dense_mfma_go<false>(a, cus, k.stream, nparts);
}

hipError_t launch_dense_mfma(const KernelCtx& k, int cus, const void* h, int B, int token_sample,
                             float tprime, uint64_t seed, float* out_logits, Part* parts,
                             int64_t* nparts) {
  MfmaArgs a{};
  a.A = k.E; a.R = k.v; a.d = k.d; a.H = static_cast<const uint16_t*>(h); a.B = B;
  a.out = out_logits; a.ld_out = k.v;
  a.token_sample = token_sample; a.tprime = tprime; a.seed = seed; a.parts = parts;
  return dense_rows_go(k, a, cus, nparts);
}

hipError_t launch_gather_shared_mfma(const KernelCtx& k, int cus, const void* h, int B,
                                     const int32_t* S, int p, int token_sample, float tprime,
                                     uint64_t seed, int32_t* out_ids, float* out_logits,
                                     Part* parts, int64_t* nparts) {
  MfmaArgs a{};
  a.A = k.Ec; a.R = (int64_t)p * k.b; a.d = k.d; a.H = static_cast<const uint16_t*>(h); a.B = B;
  a.out = out_logits; a.ld_out = a.R; a.out_ids = out_ids;
  a.token_sample = token_sample; a.tprime = tprime; a.seed = seed; a.parts = parts;
  a.rows_map = S; a.bsz = (int)k.b; a.c2t = k.c2t;
  return mfma_dispatch<0, true>(a, cus, k.stream, nparts);
}

hipError_t launch_spec_mfma(const KernelCtx& k, int cus, const void* h, int B, float T,
                            uint64_t seed, const int32_t* t2c, const uint32_t* bits, int W,
                            Part* parts, int64_t* nparts) {
  MfmaArgs a{};
  a.A = k.E; a.R = k.v; a.d = k.d; a.H = static_cast<const uint16_t*>(h); a.B = B;
  a.token_sample = 0; a.tprime = T; a.seed = seed; a.parts = parts;
  a.t2c = t2c; a.bits = bits; a.W = W;
  return dense_rows_go(k, a, cus, nparts);
}

}  // namespace fh
