// gemv_a8.hpp -- MXFP4 weights times 8-bit activations (W4A8, the Ling-3.0 MoE
// article's measured configuration, sec. 5-6) on the scaled matrix cores of
// gfx950: v_mfma_scale_f32_16x16x128_f8f6f4 with the activations as the FP8
// E4M3 A operand and the weights as the FP4 E2M1 B operand, both with their own
// E8M0 scale per 32 K, applied by the instruction.
//
//  * Staging: each workgroup quantises its input range to MXFP8 in LDS -- per
//    vector and 32 columns the smallest power of two 2^e with amax / 2^e <= 448
//    (E4M3's largest value, so nothing saturates), elements E4M3 of x / 2^e
//    rounded to nearest even -- codes [M][chunks * 256] and scales
//    [M][chunks * 8], zero past d_in.
//  * Operand layouts of the instruction (measured on the device): B lane i holds
//    column i % 16 (a weight row), K 32 (i / 16) .. +31 in its first 4 dwords --
//    one packed slot after the 16-lane-group transpose (once per dword); A lane
//    i holds row i % 16 (a vector) with K 16 (i / 16) .. +15 in bytes 0-15 and
//    K 64 + 16 (i / 16) .. +15 in bytes 16-31; the scale of lane i applies to K
//    block i / 16 of its row or column.
//  * One MFMA per 16-row block and half tile (4 slots = K 128), accumulating in
//    place: no conversion and no scale arithmetic on the VALU.
//  * Gate and up (NMAT = 2, the fused SiLU epilogue): one staging serves both
//    matrices; the items alternate matrices as in the bf16 matrix-core kernel.
//  * Mixture-of-experts modes (the article's measured W4A8 MoE, Table 1 and
//    sec. 3), as in the bf16 matrix-core kernel: MODE 1, gate/up over the
//    union's slots (the slot's expert from the routing table); MODE 2, down with
//    K over the union's (slot, chunk)s, each slot's h quantised to MXFP8 in the
//    staging like any input, each chunk's product weighted per token by the
//    slot's coefficient (the MFMA's result is added to the accumulators through
//    one FMA per value, since a coefficient is no power of two).
// The split-K tree and the epilogues are those of the other kernels.
#pragma once
#include "gemv_mfma.hpp"

namespace fp4g {

typedef int i32x8 __attribute__((ext_vector_type(8)));

// LDS of a launch: codes + scales of M vectors (rows padded by 64 bytes), then a
// zero area of one window, or the reduction buffer where that is larger.
inline size_t a8_lds_bytes(const Plan& pl, int M, int nmat) {
  const size_t staged = (size_t)M * (pl.wg_chunks * 264 + kXPad) + kZeroBytes;
  const size_t red = (size_t)kWavesPerWg * 16 * nmat * 64 * 4;
  return staged > red ? staged : red;
}

// Four waves per SIMD (128 registers per lane): every form fits without spills.
template <int M, int NMAT, int EPI, int MODE = 0>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4))) void k_gemv_a8(GemvParams p, MfmaMoe q) {
  static_assert((NMAT == 1 && EPI == EPI_STORE) || (NMAT == 2 && EPI == EPI_SILU), "A8: plain or gate/up");
  constexpr bool MOE = MODE == 1, MOED = MODE == 2;
  static_assert((!MOE || NMAT == 2) && (!MOED || NMAT == 1), "MoE modes: gate/up, down");
  // values per lane at the end: matrix a, rows 16 r + cl, vectors 4 kg + v
  constexpr int NV = 16 * NMAT;
  constexpr int TILE = kTileMx;
  extern __shared__ __attribute__((aligned(16))) uint8_t xs[];
  float(*red)[NV][64] = reinterpret_cast<float(*)[NV][64]>(xs);  // after the products

  const int lane = threadIdx.x & 63;
  const int wave = wave_id();
  const int gt = uniform(blockIdx.x / p.S);
  const int s = uniform(blockIdx.x % p.S);
  const int mem = MOE ? 0 : member_of(p, gt);
  int g = gt - p.gbase[mem];
  const uint8_t* w0 = p.w[mem];
  const uint8_t* w1 = p.w[NMAT - 1];  // up (NMAT = 2; the group has one member)
  int slot = 0, expert = 0;
  if constexpr (MOE) {
    slot = uniform(gt / q.rg);
    g = gt - slot * q.rg;
    if (slot >= q.route[0]) return;  // past the realised union: no byte read
    expert = q.route[1 + slot];
    w0 = expert >= 0 ? p.w[0] + (uint64_t)expert * q.stride[0] : q.sh[0];
    w1 = expert >= 0 ? p.w[1] + (uint64_t)expert * q.stride[1] : q.sh[1];
  }
  const int wg_c0 = s * p.wg_chunks;
  const int wg_c1 = min(p.C, wg_c0 + p.wg_chunks);
  const int per_wave = (wg_c1 - wg_c0 + kWavesPerWg - 1) / kWavesPerWg;
  int c0 = min(wg_c1, wg_c0 + wave * per_wave);
  int c1 = min(wg_c1, c0 + per_wave);
  int n_valid = p.C;  // chunks that carry data (down: those of the realised union)
  if constexpr (MOED) {
    n_valid = uniform(q.route[0]) * q.cd;
    c1 = min(c1, n_valid);
    c0 = min(c0, c1);
  }
  const int cl = lane & 15, kg = lane >> 4;
  const int64_t tile0 = (int64_t)g * (MOED ? q.cd : p.C);
  // items (chunk, half, matrix), matrix fastest
  auto item_tile = [&](int it) {
    const int cv = c0 + it / (2 * NMAT);
    if constexpr (MOED) {
      const int sl = cv / q.cd, e = q.route[1 + sl];
      const uint8_t* base = e >= 0 ? p.w[0] + (uint64_t)e * q.stride[0] : q.sh[0];
      return base + (tile0 + (cv - sl * q.cd)) * TILE;
    }
    return (it % NMAT ? w1 : w0) + (tile0 + cv) * TILE;
  };
  auto item_half = [&](int it) { return (it / NMAT) & 1; };

  const int n_items = (c1 - c0) * 2 * NMAT;
  MFrag<FP4G_MXFP4> fa, fb;
  if (n_items > 0) load_mfrag<FP4G_MXFP4>(fa, item_tile(0), 0, lane);

  // staging: codes of vector m at m * cstride, its scales at sbase + m * sstride
  const int cstride = p.wg_chunks * 256 + kXPad;
  const int sbase = M * cstride, sstride = p.wg_chunks * 8;
  const int zbase = sbase + M * sstride + ((16 - (M * sstride) % 16) % 16);  // 16-B aligned zero area
  {
    const int nblk = M * p.wg_chunks * 8;  // 32-column blocks
    for (int b = threadIdx.x; b < nblk; b += kThreads) {
      const int m = b / (p.wg_chunks * 8), j = b - m * (p.wg_chunks * 8);
      u32x4 v[4] = {};
      if constexpr (MOED) {
        // chunk cv of the union: columns of slot cv / cd's h (zero past d_ff and
        // past the union)
        const int cv = wg_c0 + j / 8, sl = cv / q.cd, col = (cv - sl * q.cd) * kChunkK + (j % 8) * 32;
        if (cv < n_valid && col < q.dff) {
#pragma unroll
          for (int k = 0; k < 4; ++k)
            v[k] = *reinterpret_cast<const u32x4*>(q.hbuf + ((int64_t)sl * M + m) * q.dff + col + 8 * k);
        }
      } else {
        const int col = wg_c0 * kChunkK + j * 32;
        if (col < p.d_in) {
#pragma unroll
          for (int k = 0; k < 4; ++k) v[k] = *reinterpret_cast<const u32x4*>(p.x + (int64_t)m * p.d_in + col + 8 * k);
        }
      }
      float amax = 0.0f;
#pragma unroll
      for (int k = 0; k < 4; ++k)
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          amax = fmaxf(amax, fabsf(__uint_as_float(v[k][d] << 16)));
          amax = fmaxf(amax, fabsf(__uint_as_float(v[k][d] & 0xffff0000u)));
        }
      int e = 0;
      if (amax > 0.0f) {
        int ex;
        const float mant = frexpf(amax, &ex);  // amax = mant 2^ex, mant in [0.5, 1)
        e = mant <= 0.875f ? ex - 9 : ex - 8;  // the smallest e with amax / 2^e <= 448 = 0.875 2^9
        e = min(max(e, -127), 127);
      }
      uint32_t out[8];
#pragma unroll
      for (int k = 0; k < 4; ++k)
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          // x / 2^e is exact (a bf16 value scaled by a power of two) and at most
          // 448 in magnitude; the hardware conversion rounds it to nearest even
          // like the element rule above (a negative value that rounds to zero
          // gives the -0 code, a zero product on the matrix cores).
          const float x0 = __builtin_amdgcn_ldexpf(__uint_as_float(v[k][d] << 16), -e);
          const float x1 = __builtin_amdgcn_ldexpf(__uint_as_float(v[k][d] & 0xffff0000u), -e);
          const uint32_t pair = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(x0, x1, 0, false) & 0xffffu;
          // columns 8k + 2d, 8k + 2d + 1 -> bytes 8k + 2d .. of the block
          const int byte = 8 * k + 2 * d;
          out[byte / 4] = (byte % 4 == 0) ? pair : (out[byte / 4] | (pair << 16));
        }
      uint8_t* dst = xs + m * cstride + j * 32;
#pragma unroll
      for (int q = 0; q < 2; ++q)
        *reinterpret_cast<u32x4*>(dst + 16 * q) = u32x4{out[4 * q], out[4 * q + 1], out[4 * q + 2], out[4 * q + 3]};
      xs[sbase + m * sstride + j] = (uint8_t)(e + 127);
    }
    if (threadIdx.x < 8) *reinterpret_cast<u32x4*>(xs + zbase + threadIdx.x * 16) = u32x4{0u, 0u, 0u, 0u};
  }
  __syncthreads();

  const bool aval = cl < M;
  f32x4 acc[NMAT][4];
#pragma unroll
  for (int a = 0; a < NMAT; ++a)
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[a][r] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  auto consume = [&](MFrag<FP4G_MXFP4>& f, int it, f32x4(&ac)[4]) {
    const int cc = c0 + it / (2 * NMAT) - wg_c0;  // chunk within the staged range
    const int h = item_half(it);                  // half: K window 128 h .. of the chunk
    // A: the lane's vector's codes (K 16 kg .. and 64 + 16 kg ..) and block scale
    const int abase = aval ? cl * cstride + cc * 256 + h * 128 : zbase;
    const u32x4 a0 = *reinterpret_cast<const u32x4*>(xs + abase + 16 * kg);
    const u32x4 a1 = *reinterpret_cast<const u32x4*>(xs + abase + 64 + 16 * kg);
    const i32x8 av = {(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3], (int)a1[0], (int)a1[1], (int)a1[2], (int)a1[3]};
    const int sa = aval ? (int)xs[sbase + cl * sstride + cc * 8 + h * 4 + kg] : 127;
    // B: slot kg of rows 16 r + cl (transpose of the four slots, one dword at a time)
    u32x4 t[4];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      t[d] = u32x4{f.q[0][d], f.q[1][d], f.q[2][d], f.q[3][d]};
      transpose_slot(t[d]);
    }
    // MoE down: the chunk's slot's coefficient of each of the lane's vectors
    float cf[4] = {1.0f, 1.0f, 1.0f, 1.0f};
    if constexpr (MOED) {
      const int sl = (cc + wg_c0) / q.cd;
#pragma unroll
      for (int v = 0; v < 4; ++v) cf[v] = 4 * kg + v < M ? q.coef[sl * M + 4 * kg + v] : 0.0f;
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const i32x8 bv = {(int)t[0][r], (int)t[1][r], (int)t[2][r], (int)t[3][r], 0, 0, 0, 0};
      const int sb = (int)((f.s[r][0] >> (8 * kg)) & 0xffu);  // block 4 h + kg of row 16 r + cl
      if constexpr (MOED) {
        const f32x4 d = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, f32x4{0.0f, 0.0f, 0.0f, 0.0f}, 0, 4,
                                                                         0, sa, 0, sb);
#pragma unroll
        for (int v = 0; v < 4; ++v) ac[r][v] = __builtin_fmaf(d[v], cf[v], ac[r][v]);
      } else {
        ac[r] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, ac[r], 0, 4, 0, sa, 0, sb);
      }
    }
  };

  // fa holds even items and fb odd ones: with NMAT = 2 gate and up
  if (n_items > 0) {
    int it = 0;
    for (; it + 2 < n_items; it += 2) {
      load_mfrag<FP4G_MXFP4>(fb, item_tile(it + 1), item_half(it + 1), lane);
      consume(fa, it, acc[0]);
      load_mfrag<FP4G_MXFP4>(fa, item_tile(it + 2), item_half(it + 2), lane);
      consume(fb, it + 1, acc[NMAT - 1]);
    }
    if (it + 1 < n_items) {
      load_mfrag<FP4G_MXFP4>(fb, item_tile(it + 1), item_half(it + 1), lane);
      consume(fa, it, acc[0]);
      consume(fb, it + 1, acc[NMAT - 1]);
    } else {
      consume(fa, it, acc[0]);
    }
  }

  __syncthreads();  // every wave is past its last read of the staging area
#pragma unroll
  for (int a = 0; a < NMAT; ++a)
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int v = 0; v < 4; ++v) red[wave][(a * 4 + r) * 4 + v][lane] = acc[a][r][v];
  __syncthreads();
  if (wave != 0) return;
  float val[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) val[i] = ((red[0][i][lane] + red[1][i][lane]) + red[2][i][lane]) + red[3][i][lane];

  // units: EPI_SILU (gate, up) of (row block r, vector 4 kg + v), unit 4 r + v;
  // EPI_STORE vectors (4 kg + 2 w, + 1) of row block r, unit 2 r + w
  constexpr int NU = EPI == EPI_SILU ? 16 : 8;
  float ua[NU], ub[NU];
  bool live[NU];
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    if constexpr (EPI == EPI_SILU) {
      ua[u] = val[u];
      ub[u] = val[16 + u];
      live[u] = 4 * kg + (u & 3) < M;
    } else {
      ua[u] = val[2 * u];
      ub[u] = val[2 * u + 1];
      live[u] = 4 * kg + 2 * (u & 1) < M;
    }
  }
  exchange_tree<NU>(p.slots, (int64_t)p.gbase[p.n] * 64, (int64_t)gt * 64 + lane, p.S, s, ua, ub, live);
  const int d_out = p.d_out[mem];
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    if (!live[u]) continue;
    if constexpr (EPI == EPI_SILU) {
      const int r = u / 4, m = 4 * kg + (u & 3), row = g * 64 + 16 * r + cl;
      if (m < M && row < d_out) {
        const float tg = MOE && expert < 0 ? q.sh_ts[0] : p.tscale[0];
        const float tu = MOE && expert < 0 ? q.sh_ts[1] : p.tscale[1];
        const uint16_t hv = f32_to_bf16_rne(silu_f32(ua[u] * tg) * (ub[u] * tu));
        p.h[((int64_t)slot * M + m) * d_out + row] = hv;
        if constexpr (MOE) {
          if (q.hdbg) {
            if (expert < 0) {
              q.hdbg[((int64_t)m * q.nh + q.k) * d_out + row] = hv;
            } else {
              for (int j = 0; j < q.k; ++j)
                if (q.ids[m * q.k + j] == expert) q.hdbg[((int64_t)m * q.nh + j) * d_out + row] = hv;
            }
          }
        }
      }
    } else {
      const int r = u / 2, w = u % 2;
      const int m = 4 * kg + 2 * w, row = g * 64 + 16 * r + cl;
      if (row < d_out) {
        float* y = p.y[mem] + row;
        if (m < M) y[(int64_t)m * d_out] = ua[u] * p.tscale[mem];
        if (m + 1 < M) y[(int64_t)(m + 1) * d_out] = ub[u] * p.tscale[mem];
      }
    }
  }
}

template <int NMAT, int EPI>
hipError_t launch_a8(int M, const GemvParams& p, unsigned grid, size_t lds, hipStream_t s) {
  switch (M) {
#define FP4G_CASE(MM)                                                   \
  case MM:                                                              \
    k_gemv_a8<MM, NMAT, EPI><<<grid, kThreads, lds, s>>>(p, MfmaMoe{}); \
    break;
    FP4G_CASE(1) FP4G_CASE(2) FP4G_CASE(3) FP4G_CASE(4) FP4G_CASE(5) FP4G_CASE(6) FP4G_CASE(7) FP4G_CASE(8)
    FP4G_CASE(9) FP4G_CASE(10) FP4G_CASE(11) FP4G_CASE(12) FP4G_CASE(13) FP4G_CASE(14) FP4G_CASE(15) FP4G_CASE(16)
#undef FP4G_CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// The W4A8 mixture-of-experts gate/up (MODE 1) and down (MODE 2), M = 1..16.
template <int MODE>
hipError_t launch_a8_moe(int M, const GemvParams& p, const MfmaMoe& q, unsigned grid, size_t lds, hipStream_t s) {
  constexpr int NMAT = MODE == 1 ? 2 : 1;
  constexpr int EPI = MODE == 1 ? EPI_SILU : EPI_STORE;
  switch (M) {
#define FP4G_CASE(MM)                                                     \
  case MM:                                                                \
    k_gemv_a8<MM, NMAT, EPI, MODE><<<grid, kThreads, lds, s>>>(p, q);     \
    break;
    FP4G_CASE(1) FP4G_CASE(2) FP4G_CASE(3) FP4G_CASE(4) FP4G_CASE(5) FP4G_CASE(6) FP4G_CASE(7) FP4G_CASE(8)
    FP4G_CASE(9) FP4G_CASE(10) FP4G_CASE(11) FP4G_CASE(12) FP4G_CASE(13) FP4G_CASE(14) FP4G_CASE(15) FP4G_CASE(16)
#undef FP4G_CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace fp4g
