// attn_norms: the precomputed norms of the Cauchy-Schwarz bound softmax
// (vatt-ghern.pages.dev "deep-heygen-avatar-iv-trillium-tpu", section
// 拿掉 softmax 的序列相依: a small set of norms is computed ahead of the
// attention kernel so every query row knows its shift before the key loop).
//
// Outputs (fp32, contiguous): q_norm[B][H][N] = |q_n|, k_gmax[B][H][N/16] =
// max |k_n| over each 16-key granule, head_max[B][H][2] = (max|q|, max|k|).
//
// HBM-bound: reads Q and K once (2*B*H*N*D*2 bytes) and writes 4*B*H*N*(1+1/16)
// bytes.  Each wave takes one 16-row granule of one head; a row of D bf16 is
// read by D/8 consecutive lanes with 16-byte loads, so one wave-wide load
// covers 64/(D/8) whole rows (coalesced, 1 KiB per instruction).  head_max is
// then reduced from q_norm and k_gmax by a second, small pass (8 workgroups a
// head): merging the maxima of thousands of workgroups by atomics on the same
// two words serialises, and costs more than this pass over 1/D of the data.
#include "bsvf_device.h"
#include "bsvf_internal.h"

namespace bsvf {
namespace {

constexpr int kNormThreads = 256;
constexpr int kGranulesPerWave = 1;

struct NormArgs {
  const u16* q;
  const u16* k;
  int64_t qs_b, qs_h, qs_n, ks_b, ks_h, ks_n;
  int32_t H, N;
  float* q_norm;
  float* k_gmax;
  float* head_max;
};

// head_max[bh] = (max_n q_norm[bh][n], max_g k_gmax[bh][g]).  Each head's rows
// are split over kHeadMaxSlices workgroups (a head's q_norm is a few hundred
// KB, and B*H workgroups alone leave most of the GPU idle); each merges its
// slice's maxima with an unsigned atomic max on the float bits (norms are >= 0,
// so the orders agree), into a head_max the producing kernel cleared.  Maxima
// are exact, so the result does not depend on order.  With VEC the q_norm rows
// (16-byte aligned) are read 16 bytes per lane.
constexpr int kHeadMaxThreads = 512;
constexpr int kHeadMaxSlices = 8;

typedef float f32x4n __attribute__((ext_vector_type(4)));

template <bool VEC>
__global__ __launch_bounds__(kHeadMaxThreads) void head_max_kernel(const float* __restrict__ q_norm,
                                                                   const float* __restrict__ k_gmax, int32_t N,
                                                                   float* __restrict__ head_max) {
  const int64_t bh = blockIdx.y;
  const float* qn = q_norm + bh * N;
  const float* kg = k_gmax + bh * (N / 16);
  const int t = blockIdx.x * kHeadMaxThreads + threadIdx.x, stride = kHeadMaxSlices * kHeadMaxThreads;
  float mq = 0.0f, mk = 0.0f;
  if constexpr (VEC) {
    const f32x4n* q4 = reinterpret_cast<const f32x4n*>(qn);
#pragma unroll 4
    for (int i = t; i < N / 4; i += stride) {
      const f32x4n v = q4[i];
      mq = fmaxf(mq, fmaxf(fmaxf(v[0], v[1]), fmaxf(v[2], v[3])));
    }
  } else {
#pragma unroll 4
    for (int i = t; i < N; i += stride) mq = fmaxf(mq, qn[i]);
  }
#pragma unroll 2
  for (int i = t; i < N / 16; i += stride) mk = fmaxf(mk, kg[i]);
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    mq = fmaxf(mq, __shfl_xor(mq, m));
    mk = fmaxf(mk, __shfl_xor(mk, m));
  }
  __shared__ float red[2][kHeadMaxThreads / 64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) { red[0][wave] = mq; red[1][wave] = mk; }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < kHeadMaxThreads / 64; ++w) { mq = fmaxf(mq, red[0][w]); mk = fmaxf(mk, red[1][w]); }
    atomicMax(reinterpret_cast<unsigned int*>(head_max + 2 * bh), __float_as_uint(mq));
    atomicMax(reinterpret_cast<unsigned int*>(head_max + 2 * bh + 1), __float_as_uint(mk));
  }
}

template <int D>
__global__ __launch_bounds__(kNormThreads) void norms_kernel(NormArgs a) {
  constexpr int LPR = D / 8;        // lanes per row (16 bytes each)
  constexpr int RPI = 64 / LPR;     // rows per wave-wide load
  constexpr int IPG = 16 / RPI;     // loads per 16-row granule
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int bh = blockIdx.y;
  const int b = bh / a.H, h = bh % a.H;
  const int G = a.N / 16;
  const u16* qh = a.q + b * a.qs_b + h * a.qs_h;
  const u16* kh = a.k + b * a.ks_b + h * a.ks_h;
  const int c = lane % LPR, rsub = lane / LPR;

  // the head-max pass that follows merges into a cleared head_max
  if (blockIdx.x == 0 && threadIdx.x < 2) a.head_max[2 * bh + threadIdx.x] = 0.0f;
  const int g0 = (blockIdx.x * (kNormThreads / 64) + wave) * kGranulesPerWave;
  // All of this wave's loads are issued before any arithmetic.  Granules past
  // the end re-read the last one (in bounds) and are not stored.
  u32x4 qv[kGranulesPerWave][IPG], kv[kGranulesPerWave][IPG];
#pragma unroll
  for (int gi = 0; gi < kGranulesPerWave; ++gi) {
    const int g = min(g0 + gi, G - 1);
#pragma unroll
    for (int it = 0; it < IPG; ++it) {
      const int row = g * 16 + it * RPI + rsub;
      qv[gi][it] = *reinterpret_cast<const u32x4*>(qh + (int64_t)row * a.qs_n + 8 * c);
      kv[gi][it] = *reinterpret_cast<const u32x4*>(kh + (int64_t)row * a.ks_n + 8 * c);
    }
  }
#pragma unroll
  for (int gi = 0; gi < kGranulesPerWave; ++gi) {
    const int g = g0 + gi;
    if (g >= G) break;
    float kg = 0.0f;
#pragma unroll
    for (int it = 0; it < IPG; ++it) {
      float sq = 0.0f, sk = 0.0f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float q0 = bf16lo(qv[gi][it][e]), q1 = bf16hi(qv[gi][it][e]);
        const float k0 = bf16lo(kv[gi][it][e]), k1 = bf16hi(kv[gi][it][e]);
        sq = fmaf(q0, q0, sq); sq = fmaf(q1, q1, sq);
        sk = fmaf(k0, k0, sk); sk = fmaf(k1, k1, sk);
      }
#pragma unroll
      for (int m = LPR / 2; m >= 1; m >>= 1) {
        sq += __shfl_xor(sq, m);
        sk += __shfl_xor(sk, m);
      }
      const float qn = __builtin_sqrtf(sq), kn = __builtin_sqrtf(sk);
      const int row = g * 16 + it * RPI + rsub;
      if (c == 0) a.q_norm[(int64_t)bh * a.N + row] = qn;
      kg = fmaxf(kg, kn);
    }
#pragma unroll
    for (int m = LPR; m < 64; m <<= 1) kg = fmaxf(kg, __shfl_xor(kg, m));
    if (lane == 0) a.k_gmax[(int64_t)bh * G + g] = kg;
  }
}

}  // namespace

int launch_head_max(const float* q_norm, const float* k_gmax, int32_t bh, int32_t n, float* head_max,
                    hipStream_t stream) {
  // N % 16 == 0, so every head's q_norm row is 16-byte aligned when the base is
  const dim3 grid(kHeadMaxSlices, bh);
  if (aligned16(q_norm))
    hipLaunchKernelGGL(head_max_kernel<true>, grid, dim3(kHeadMaxThreads), 0, stream, q_norm, k_gmax, n, head_max);
  else
    hipLaunchKernelGGL(head_max_kernel<false>, grid, dim3(kHeadMaxThreads), 0, stream, q_norm, k_gmax, n, head_max);
  return 0;
}

}  // namespace bsvf

using namespace bsvf;

extern "C" int attn_norms(const void* q, const void* k, int32_t batch, int32_t heads,
                          int32_t seq_len, int32_t head_dim, const int64_t* q_strides,
                          const int64_t* k_strides, float* q_norm, float* k_gmax,
                          float* head_max, hipStream_t stream) {
  if (batch <= 0 || heads <= 0 || seq_len <= 0) return fail(ATTN_E_INVAL, "sizes must be positive");
  if (head_dim != 64 && head_dim != 128) return fail(ATTN_E_UNSUPPORTED, "head_dim must be 64 or 128");
  if (seq_len % 16) return fail(ATTN_E_ALIGN, "seq_len must be a multiple of 16");
  int st;
  if ((st = check_tensor("q", q, q_strides, batch, heads, seq_len, head_dim))) return st;
  if ((st = check_tensor("k", k, k_strides, batch, heads, seq_len, head_dim))) return st;
  if (!q_norm || !k_gmax || !head_max) return fail(ATTN_E_INVAL, "output pointers must not be NULL");
  if ((int64_t)batch * heads > 65535) return fail(ATTN_E_SIZE, "batch * heads exceeds 65535");
  if ((int64_t)batch * heads * seq_len > (int64_t)1 << 40) return fail(ATTN_E_SIZE, "too many rows");

  NormArgs a;
  a.q = static_cast<const u16*>(q);
  a.k = static_cast<const u16*>(k);
  a.qs_b = q_strides[0]; a.qs_h = q_strides[1]; a.qs_n = q_strides[2];
  a.ks_b = k_strides[0]; a.ks_h = k_strides[1]; a.ks_n = k_strides[2];
  a.H = heads;
  a.N = seq_len;
  a.q_norm = q_norm;
  a.k_gmax = k_gmax;
  a.head_max = head_max;

  const int granules = seq_len / 16;
  const int per_block = (kNormThreads / 64) * kGranulesPerWave;
  dim3 grid((granules + per_block - 1) / per_block, batch * heads);
  if (head_dim == 128)
    hipLaunchKernelGGL(norms_kernel<128>, grid, dim3(kNormThreads), 0, stream, a);
  else
    hipLaunchKernelGGL(norms_kernel<64>, grid, dim3(kNormThreads), 0, stream, a);
  launch_head_max(q_norm, k_gmax, batch * heads, seq_len, head_max, stream);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(ATTN_E_HIP, std::string("launch failed: ") + hipGetErrorString(e));
  return bsvf::ok();
}
