// attn_fwd: forward pass of frame-aligned block-sparse attention on gfx950.
//
// The method (vatt-ghern.pages.dev "deep-heygen-avatar-iv-trillium-tpu",
// sections 把 block 縮到 16 and 拿掉 softmax 的序列相依; bytechap "How it
// works"; cloudcurated Wall 2 and Wall 3):
//   * the key set of a query tile is a list of intervals whose ends are
//     multiples of 16 tokens on frame edges, so every key block is either
//     fully attended or absent: no mask predicate, no padding, no extra scan;
//   * softmax either keeps the standard running max (rescaling the running
//     sum and accumulator whenever the max grows), or fixes each row's shift
//     before the key loop to the Cauchy-Schwarz bound scale*|q_i|*max|k_j|
//     from precomputed norms, so the loop never rescales; heads whose bound
//     is too loose take the running-max path inside the same kernel.
//
// gfx950 design (not the TPU kernel's):
//   * One workgroup per query tile (<= 256 rows), 4 waves x 64 query rows.
//     A wave holds its Q rows in VGPRs for the whole tile.
//   * S^T = K * Q^T and O^T = V^T * P^T with v_mfma_f32_32x32x16_bf16 (fp32
//     accumulate).  With that orientation lane (n, h) of a 32x32 accumulator
//     owns query n and 16 of the 32 keys (or 16 of the 32 output dims), so
//     the row shift, the row sum and the rescale factor of a query all live
//     in the lanes that own that query: P feeds the second MFMA straight from
//     registers, and the bound path needs no cross-lane traffic at all.
//   * K and V^T stages of 64 keys are staged in LDS, double-buffered, with the
//     next stage's global loads in flight during the current stage's math.
//     16-byte chunks are XOR-swizzled so MFMA operand reads are free of bank
//     conflicts; V is transposed while being written to LDS (keys contiguous
//     per output dim) so its MFMA operand is one 16-byte LDS read.
//   * Key tails of 16 tokens use a half-block path chosen per block (the
//     block's valid count is uniform), never a per-element mask.
//   * exp is v_exp_f32 on s*scale*log2(e) - m (one FMA + one exp per score).
#include "bsvf_device.h"
#include "bsvf_internal.h"

namespace bsvf {
namespace {

constexpr int BK = 64;  // keys per LDS stage
#ifndef ONLINE_NQB
#define ONLINE_NQB 1
#define ONLINE_NW 8
#endif
#ifndef BOUND_NQB
#define BOUND_NQB 1
#define BOUND_NW 8
#endif
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// Keeps the fp32 bound above every fp32-computed score: the dot-product and
// norm rounding errors are below D * 2^-24 relative for D <= 128.
constexpr float kBoundMargin = 1.0f + 1.0f / 4096.0f;

struct FwdArgs {
  const u16* q;
  const u16* k;
  const u16* v;
  u16* o;
  float* lse;
  float* shift_out;
  int64_t sq[3], sk[3], sv[3], so[3];
  int32_t B, H, N;
  float scale;
  float c2;  // scale * log2(e)
  const int32_t* q_tiles;
  const int32_t* kv_ptr;
  const int32_t* kv_iv;
  int32_t n_qt, nnz, block_q;
  const int32_t* work_order;
  int32_t n_work;
  const float* q_norm;
  const float* k_gmax;
  const float* head_max;
  int32_t mode;
  int32_t* head_path_out;
};


__device__ __forceinline__ bf16x8 to_bf16x8(const float* p) {
  bf16x8 r;
#pragma unroll
  for (int i = 0; i < 8; i += 2) {
    f32x2 f = {p[i], p[i + 1]};
    bf16x2 b = __builtin_convertvector(f, bf16x2);
    r[i] = b[0];
    r[i + 1] = b[1];
  }
  return r;
}

__device__ __forceinline__ bool interval_ok(int ks, int kl, int N) {
  return ks >= 0 && kl > 0 && ((ks | kl) & 15) == 0 && ks <= N - kl;
}

template <int D, int NQB, int NW>
struct Cfg {
  static constexpr int NT = 64 * NW;
  static constexpr int BQ = 32 * NQB * NW;
  static constexpr int DC = D / 8;               // 16-byte chunks per K row
  static constexpr int KSTEPS = D / 16;          // MFMA k-steps of Q*K^T
  static constexpr int DBLK = D / 32;            // 32-wide output blocks
  static constexpr int STAGE = 2 * BK * D;       // K + V^T elements per stage
  static constexpr int K_LOADS = BK * DC / NT;   // 16-byte K loads per thread
  static constexpr int KPT = BK * D / (NT * 8);  // V keys per thread
  static_assert(K_LOADS >= 1 && KPT >= 1 && KPT <= 4 && (4 % KPT) == 0, "tile shape");
};

// Global -> registers -> LDS staging of one 64-key stage.  Keys past the
// stage's valid count re-load the last valid key (always in bounds and finite);
// their probabilities are zeroed before they can contribute.
template <int D, int NQB, int NW>
struct Stager {
  using C = Cfg<D, NQB, NW>;
  u32x4 kr[C::K_LOADS];
  u32x4 vr[C::KPT];

  __device__ __forceinline__ void load(const u16* kh, const u16* vh, int ksn, int vsn,
                                       int start, int nvalid, int tid) {
#pragma unroll
    for (int it = 0; it < C::K_LOADS; ++it) {
      const int idx = it * C::NT + tid;
      const int key = min(idx / C::DC, nvalid - 1), c = idx % C::DC;
      kr[it] = *reinterpret_cast<const u32x4*>(kh + (start + key) * ksn + 8 * c);
    }
    const int dg = tid % C::DC, kg = tid / C::DC;
#pragma unroll
    for (int j = 0; j < C::KPT; ++j) {
      const int key = min(kg * C::KPT + j, nvalid - 1);
      vr[j] = *reinterpret_cast<const u32x4*>(vh + (start + key) * vsn + 8 * dg);
    }
  }

  __device__ __forceinline__ void store(u16* ks, u16* vt, int tid) const {
#pragma unroll
    for (int it = 0; it < C::K_LOADS; ++it) {
      const int idx = it * C::NT + tid;
      const int key = idx / C::DC, c = idx % C::DC;
      *reinterpret_cast<u32x4*>(ks + key * D + ((c ^ (key & (C::DC - 1))) << 3)) = kr[it];
    }
    // V^T: row d holds the stage's 64 keys.  Inside each 16-key group the
    // 4-key subgroups sit in the order 0, 2, 1, 3, so that the 8 keys one
    // lane half feeds to the P*V MFMA are contiguous; 16-byte chunks of a row
    // are XOR-swizzled by (d ^ d>>3) & 7.
    const int dg = tid % C::DC, kg = tid / C::DC;
    const int key0 = kg * C::KPT;
    const int s4 = (key0 >> 2) & 3;
    const int pos = (key0 & ~15) + 4 * (((s4 & 1) << 1) | (s4 >> 1)) + (key0 & 3);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int d = 8 * dg + e;
      const int off = d * BK + ((((pos >> 3) ^ (d ^ (d >> 3))) & 7) << 3) + (pos & 7);
      uint32_t h[C::KPT];
#pragma unroll
      for (int j = 0; j < C::KPT; ++j) {
        const uint32_t w = vr[j][e >> 1];
        h[j] = (e & 1) ? (w >> 16) : (w & 0xffffu);
      }
      if constexpr (C::KPT == 4) {
        u32x2 pk = {h[0] | (h[1] << 16), h[2] | (h[3] << 16)};
        *reinterpret_cast<u32x2*>(vt + off) = pk;
      } else if constexpr (C::KPT == 2) {
        *reinterpret_cast<uint32_t*>(vt + off) = h[0] | (h[1] << 16);
      } else {
        vt[off] = (u16)h[0];
      }
    }
  }
};

template <int D, int NQB, int NW>
struct Tile {
  using C = Cfg<D, NQB, NW>;
  bf16x8 qreg[NQB][C::KSTEPS];
  f32x16 oacc[NQB][C::DBLK];
  float m2[NQB];    // row shift in log2 units (bound: fixed; online: running max)
  float lsum[NQB];  // this lane half's share of the row sum
  int n, hh;

  // One LDS stage: 64 keys of which the first `nvalid` (16, 32, 48 or 64) are
  // real.  The same MFMAs run for every stage; a short stage only zeroes the
  // probabilities of its missing keys.
  template <bool BOUND>
  __device__ __forceinline__ void stage(const u16* ks, const u16* vt, int nvalid, float c2) {
    f32x16 s[2][NQB];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[kb][qb][r] = 0.0f;
    // S^T = K * Q^T: lane (n, hh) gets keys 32kb + 8i + 4hh + j (register
    // 4i + j) of query n.
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int key = 32 * kb + n;
#pragma unroll
      for (int st = 0; st < C::KSTEPS; ++st) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(ks + key * D + (((2 * st + hh) ^ (key & (C::DC - 1))) << 3));
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb)
          s[kb][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[qb][st], s[kb][qb], 0, 0, 0);
      }
    }
    bf16x8 pk[NQB][2][2];
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      if constexpr (!BOUND) {
        // Running max over the stage (missing keys hold copies of a real key of
        // this row, so they cannot raise the max above a real score).
        float mx = s[0][qb][0];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][qb][r]);
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float mnew = fmaxf(m2[qb], mx * c2);
        const float alpha = __builtin_amdgcn_exp2f(m2[qb] - mnew);
        m2[qb] = mnew;
        lsum[qb] *= alpha;
        if (__any(alpha != 1.0f)) {
#pragma unroll
          for (int db = 0; db < C::DBLK; ++db) oacc[qb][db] *= alpha;
        }
      }
      const float nm = -m2[qb];
      float p[2][16];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) p[kb][r] = __builtin_amdgcn_exp2f(fmaf(s[kb][qb][r], c2, nm));
      if (nvalid < BK) {
        // keys 32kb + 8i .. +7 are all real or all missing (16-key granules)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (32 * kb + 8 * i >= nvalid)
#pragma unroll
              for (int j = 0; j < 4; ++j) p[kb][4 * i + j] = 0.0f;
      }
      float t0 = 0.0f, t1 = 0.0f, t2 = 0.0f, t3 = 0.0f;
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        t0 += p[0][r]; t1 += p[0][r + 1]; t2 += p[1][r]; t3 += p[1][r + 1];
      }
      lsum[qb] += (t0 + t1) + (t2 + t3);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        pk[qb][kb][0] = to_bf16x8(p[kb]);
        pk[qb][kb][1] = to_bf16x8(p[kb] + 8);
      }
    }
    // O^T += V^T * P^T: k-step (kb, kst) covers keys 32kb + 16kst + [0, 16).
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int kst = 0; kst < 2; ++kst)
#pragma unroll
        for (int db = 0; db < C::DBLK; ++db) {
          const int d = 32 * db + n;
          const int chunk = 2 * (2 * kb + kst) + hh;
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(vt + d * BK + ((chunk ^ ((d ^ (d >> 3)) & 7)) << 3));
#pragma unroll
          for (int qb = 0; qb < NQB; ++qb)
            oacc[qb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pk[qb][kb][kst], oacc[qb][db], 0, 0, 0);
        }
  }
};

template <int D, int NQB, int NW, bool BOUND>
__device__ __forceinline__ void run_tile(const FwdArgs& a, const int32_t* __restrict__ kv_iv, u16* smem,
                                         Tile<D, NQB, NW>& T, const u16* kh, const u16* vh,
                                         int e0, int e1, int tid) {
  using C = Cfg<D, NQB, NW>;
  const int ksn = (int)a.sk[2], vsn = (int)a.sv[2];
  // Walk the tile's intervals in stages of up to 64 keys.
  int e = e0;
  while (e < e1 && !interval_ok(kv_iv[2 * e], kv_iv[2 * e + 1], a.N)) ++e;
  if (e >= e1) return;
  int cs = kv_iv[2 * e], cl = kv_iv[2 * e + 1];  // current interval
  int off = 0;
  Stager<D, NQB, NW> sg;
  int cur_n = min(BK, cl);
  sg.load(kh, vh, ksn, vsn, cs, cur_n, tid);
  sg.store(smem, smem + BK * D, tid);
  __syncthreads();
  int buf = 0;
  while (true) {
    int noff = off + BK, ncs = cs, ncl = cl, ne = e;
    bool has_next = true;
    if (noff >= cl) {
      noff = 0;
      ++ne;
      while (ne < e1 && !interval_ok(kv_iv[2 * ne], kv_iv[2 * ne + 1], a.N)) ++ne;
      if (ne >= e1) has_next = false;
      else { ncs = kv_iv[2 * ne]; ncl = kv_iv[2 * ne + 1]; }
    }
    const int next_n = has_next ? min(BK, ncl - noff) : 0;
    if (has_next) sg.load(kh, vh, ksn, vsn, ncs + noff, next_n, tid);
    u16* ks = smem + buf * C::STAGE;
    T.template stage<BOUND>(ks, ks + BK * D, cur_n, a.c2);
    if (!has_next) break;
    u16* nks = smem + (buf ^ 1) * C::STAGE;
    sg.store(nks, nks + BK * D, tid);
    __syncthreads();
    buf ^= 1;
    e = ne; cs = ncs; cl = ncl; off = noff; cur_n = next_n;
  }
}

// BOUND selects the softmax path this instantiation runs.  Both are launched
// over the same work; a workgroup whose head takes the other path exits at
// once, so each head is computed by exactly one of them and each path gets a
// register allocation of its own.
template <int D, int NQB, int NW, bool BOUND>
__global__ __launch_bounds__(64 * NW) void fwd_kernel(FwdArgs a, const int32_t* __restrict__ q_tiles,
                                                      const int32_t* __restrict__ kv_ptr,
                                                      const int32_t* __restrict__ kv_iv,
                                                      const int32_t* __restrict__ work_order,
                                                      const float* __restrict__ k_gmax,
                                                      const float* __restrict__ head_max) {
  using C = Cfg<D, NQB, NW>;
  __shared__ __attribute__((aligned(16))) u16 smem[2 * C::STAGE];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  int w = blockIdx.x;
  if (work_order) {
    if (w >= a.n_work) return;
    w = work_order[w];
  }
  const int total = a.n_qt * a.H * a.B;
  if (w < 0 || w >= total) return;
  const int tile = w % a.n_qt, bh = w / a.n_qt;
  const int b = bh / a.H, h = bh % a.H;
  const int qs = q_tiles[2 * tile], nr = q_tiles[2 * tile + 1];
  if (qs < 0 || nr <= 0 || nr > C::BQ || nr > a.block_q || qs > a.N - nr) return;
  int e0 = kv_ptr[tile], e1 = kv_ptr[tile + 1];
  e0 = max(0, min(e0, a.nnz));
  e1 = max(e0, min(e1, a.nnz));

  // Head path: uniform per workgroup.
  bool bound = false;
  if (a.mode == ATTN_SOFTMAX_BOUND_FORCED) {
    bound = true;
  } else if (a.mode == ATTN_SOFTMAX_BOUND) {
    const float mq = head_max[2 * bh], mk = head_max[2 * bh + 1];
    bound = 2.0f * a.scale * mq * mk <= ATTN_ELIGIBLE_NATS;
  }
  if (bound != BOUND) return;
  if (tile == 0 && tid == 0 && a.head_path_out) a.head_path_out[bh] = bound ? ATTN_PATH_BOUND : ATTN_PATH_ONLINE;

  // Tile-wide max key norm over every attended 16-key granule (bound only).
  float kfac = 0.0f;
  if constexpr (BOUND) {
    float km = 0.0f;
    const float* kg = k_gmax + (int64_t)bh * (a.N / 16);
    for (int e = e0; e < e1; ++e) {
      const int ks = kv_iv[2 * e], kl = kv_iv[2 * e + 1];
      if (!interval_ok(ks, kl, a.N)) continue;
      for (int g = ks / 16 + tid; g < (ks + kl) / 16; g += C::NT) km = fmaxf(km, kg[g]);
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) km = fmaxf(km, __shfl_xor(km, m));
    float* red = reinterpret_cast<float*>(smem + C::STAGE);
    if (lane == 0) red[wave] = km;
    __syncthreads();
    km = red[0];
#pragma unroll
    for (int i = 1; i < NW; ++i) km = fmaxf(km, red[i]);
    kfac = a.scale * km * kBoundMargin;
  }

  Tile<D, NQB, NW> T;
  T.n = lane & 31;
  T.hh = lane >> 5;
  const int row0 = wave * 32 * NQB;
  const u16* qh = a.q + b * a.sq[0] + h * a.sq[1];
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) {
    const int r = row0 + qb * 32 + T.n;
    const bool valid = r < nr;
    const u16* qp = qh + (int64_t)(qs + (valid ? r : 0)) * a.sq[2];
#pragma unroll
    for (int st = 0; st < C::KSTEPS; ++st) {
      bf16x8 z = {};
      const bf16x8 x = *reinterpret_cast<const bf16x8*>(qp + 16 * st + 8 * T.hh);
      T.qreg[qb][st] = valid ? x : z;
    }
    if constexpr (BOUND) {
      const float qn = a.q_norm[(int64_t)bh * a.N + qs + (valid ? r : 0)];
      T.m2[qb] = valid ? qn * kfac * kLog2e : 0.0f;
    } else {
      T.m2[qb] = -INFINITY;
    }
    T.lsum[qb] = 0.0f;
#pragma unroll
    for (int db = 0; db < C::DBLK; ++db)
#pragma unroll
      for (int r2 = 0; r2 < 16; ++r2) T.oacc[qb][db][r2] = 0.0f;
  }

  const u16* kh = a.k + b * a.sk[0] + h * a.sk[1];
  const u16* vh = a.v + b * a.sv[0] + h * a.sv[1];
  run_tile<D, NQB, NW, BOUND>(a, kv_iv, smem, T, kh, vh, e0, e1, tid);

  // Epilogue: O = O_acc / l (bf16, nearest even), LSE = m + ln l.
  u16* oh = a.o + b * a.so[0] + h * a.so[1];
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) {
    const float lt = T.lsum[qb] + __shfl_xor(T.lsum[qb], 32);
    const int r = row0 + qb * 32 + T.n;
    if (r >= nr) continue;
    const float inv = 1.0f / lt;
    u16* op = oh + (int64_t)(qs + r) * a.so[2];
#pragma unroll
    for (int db = 0; db < C::DBLK; ++db) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        f32x2 f0 = {T.oacc[qb][db][4 * i] * inv, T.oacc[qb][db][4 * i + 1] * inv};
        f32x2 f1 = {T.oacc[qb][db][4 * i + 2] * inv, T.oacc[qb][db][4 * i + 3] * inv};
        bf16x2 b0 = __builtin_convertvector(f0, bf16x2), b1 = __builtin_convertvector(f1, bf16x2);
        u32x2 pk = {__builtin_bit_cast(uint32_t, b0), __builtin_bit_cast(uint32_t, b1)};
        *reinterpret_cast<u32x2*>(op + 32 * db + 8 * i + 4 * T.hh) = pk;
      }
    }
    if (T.hh == 0) {
      const int64_t ri = (int64_t)bh * a.N + qs + r;
      if (a.lse) a.lse[ri] = (T.m2[qb] + __builtin_amdgcn_logf(lt)) * kLn2;
      if (a.shift_out) a.shift_out[ri] = T.m2[qb] * kLn2;
    }
  }
}

template <int D, int NQB, int NW, bool BOUND>
int launch(const FwdArgs& a, int grid, hipStream_t stream) {
  hipLaunchKernelGGL((fwd_kernel<D, NQB, NW, BOUND>), dim3(grid), dim3(64 * NW), 0, stream, a,
                     a.q_tiles, a.kv_ptr, a.kv_iv, a.work_order, a.k_gmax, a.head_max);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(ATTN_E_HIP, std::string("launch failed: ") + hipGetErrorString(e));
  return ok();
}

}  // namespace
}  // namespace bsvf

using namespace bsvf;

extern "C" int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                        float* shift_out, int32_t batch, int32_t heads, int32_t seq_len,
                        int32_t head_dim, const int64_t* strides, float scale,
                        const attn_blocks_t* blocks, const float* q_norm, const float* k_gmax,
                        const float* head_max, int32_t softmax_mode, int32_t* head_path_out,
                        hipStream_t stream) {
  if (batch <= 0 || heads <= 0 || seq_len <= 0) return fail(ATTN_E_INVAL, "sizes must be positive");
  if (head_dim != 64 && head_dim != 128) return fail(ATTN_E_UNSUPPORTED, "head_dim must be 64 or 128");
  if (seq_len % 16) return fail(ATTN_E_ALIGN, "seq_len must be a multiple of 16");
  if (!strides) return fail(ATTN_E_INVAL, "strides is NULL");
  if (!(scale > 0.0f) || !(scale < 3.0e38f)) return fail(ATTN_E_INVAL, "scale must be positive and finite");
  if (softmax_mode < ATTN_SOFTMAX_ONLINE || softmax_mode > ATTN_SOFTMAX_BOUND_FORCED)
    return fail(ATTN_E_INVAL, "bad softmax_mode");
  int st;
  if ((st = check_tensor("q", q, strides + 0, batch, heads, seq_len, head_dim))) return st;
  if ((st = check_tensor("k", k, strides + 3, batch, heads, seq_len, head_dim))) return st;
  if ((st = check_tensor("v", v, strides + 6, batch, heads, seq_len, head_dim))) return st;
  if ((st = check_tensor("o", o, strides + 9, batch, heads, seq_len, head_dim))) return st;
  if (!blocks) return fail(ATTN_E_INVAL, "blocks is NULL");
  if (!blocks->q_tiles || !blocks->kv_ptr || !blocks->kv_iv) return fail(ATTN_E_INVAL, "block list pointers are NULL");
  if (blocks->n_qt <= 0 || blocks->nnz <= 0) return fail(ATTN_E_INVAL, "n_qt and nnz must be positive");
  if (blocks->block_q <= 0 || blocks->block_q % 16) return fail(ATTN_E_ALIGN, "block_q must be a positive multiple of 16");
  if (blocks->block_q > ATTN_MAX_BLOCK_Q) return fail(ATTN_E_UNSUPPORTED, "block_q exceeds ATTN_MAX_BLOCK_Q");
  if (blocks->work_order && blocks->n_work <= 0) return fail(ATTN_E_INVAL, "n_work must be positive");
  if (softmax_mode != ATTN_SOFTMAX_ONLINE && (!q_norm || !k_gmax || !head_max))
    return fail(ATTN_E_UNSUPPORTED, "bound softmax needs q_norm, k_gmax and head_max");
  const int64_t items = (int64_t)blocks->n_qt * heads * batch;
  if (items > 2147483647LL) return fail(ATTN_E_SIZE, "too many work items");
  if ((int64_t)batch * heads * seq_len > 2147483647LL) return fail(ATTN_E_SIZE, "B*H*N exceeds INT32_MAX");

  FwdArgs a;
  a.q = static_cast<const u16*>(q);
  a.k = static_cast<const u16*>(k);
  a.v = static_cast<const u16*>(v);
  a.o = static_cast<u16*>(o);
  a.lse = lse;
  a.shift_out = shift_out;
  for (int i = 0; i < 3; ++i) {
    a.sq[i] = strides[i];
    a.sk[i] = strides[3 + i];
    a.sv[i] = strides[6 + i];
    a.so[i] = strides[9 + i];
  }
  a.B = batch;
  a.H = heads;
  a.N = seq_len;
  a.scale = scale;
  a.c2 = scale * kLog2e;
  a.q_tiles = blocks->q_tiles;
  a.kv_ptr = blocks->kv_ptr;
  a.kv_iv = blocks->kv_iv;
  a.n_qt = blocks->n_qt;
  a.nnz = blocks->nnz;
  a.block_q = blocks->block_q;
  a.work_order = blocks->work_order;
  a.n_work = blocks->work_order ? blocks->n_work : 0;
  a.q_norm = q_norm;
  a.k_gmax = k_gmax;
  a.head_max = head_max;
  a.mode = softmax_mode;
  a.head_path_out = head_path_out;

  const int grid = blocks->work_order ? blocks->n_work : (int)items;
  if (softmax_mode != ATTN_SOFTMAX_ONLINE) {
    st = head_dim == 128 ? launch<128, BOUND_NQB, BOUND_NW, true>(a, grid, stream)
                         : launch<64, BOUND_NQB, BOUND_NW, true>(a, grid, stream);
    if (st) return st;
  }
  if (softmax_mode != ATTN_SOFTMAX_BOUND_FORCED) {
    st = head_dim == 128 ? launch<128, ONLINE_NQB, ONLINE_NW, false>(a, grid, stream)
                         : launch<64, ONLINE_NQB, ONLINE_NW, false>(a, grid, stream);
    if (st) return st;
  }
  return ok();
}
