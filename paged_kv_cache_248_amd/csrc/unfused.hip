// Unfused causal paged prefill: the standard three-step attention that the
// fused kernel replaces.  Per sequence, the score matrix S = scale * Q K^T
// (fp32) and the softmax P (input dtype) are written to HBM in full and read
// back, as in the plain attention that [P-wall] section 二.1 describes as
// holding the N x N intermediate in HBM and that [P-opt]'s FlashAttention
// comparison table ("传统Attention" column: P stored, several separate
// kernels) takes as the starting point.
//
// Steps for one sequence b (q new tokens, n keys, prefix n - q):
//   1. gather: K and V of tokens [0, n) through the block table into
//      contiguous [Hkv, n, D]; the q query rows regrouped to [Hkv, q, G, D]
//      so that every GQA group is one matrix of q*G rows;
//   2. S_g = scale * Q_g K_g^T, fp32 [q*G, n] per kv head (hipBLASLt,
//      strided batch over the kv heads);
//   3. row softmax of S with the causal mask (row t sees keys 0..n-q+t),
//      written as P in the input dtype, masked entries 0;
//   4. O_g = P_g V_g (hipBLASLt, fp32 accumulation, input dtype out);
//   5. scatter the O rows back to the packed [T, Hq, D] output.
// The GEMMs are vendor library calls on purpose: the point is the cost of
// the S/P round trips, not a hand-tuned matrix kernel.
#include <hip/hip_runtime.h>
#include <hipblaslt/hipblaslt.h>

#include <map>
#include <mutex>
#include <tuple>

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ int64_t grid_stride_start() {
  return (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
}
__device__ __forceinline__ int64_t grid_stride() { return (int64_t)gridDim.x * blockDim.x; }

// K and V rows of logical tokens [0, n) of one sequence -> [Hkv, n, row].
// A row is `row_chunks` 16-byte pieces; block ids are clamped into the pool.
__global__ __launch_bounds__(kThreads) void unfused_gather_kv_kernel(
    const u32x4 *__restrict__ k_cache, const u32x4 *__restrict__ v_cache,
    u32x4 *__restrict__ kg, u32x4 *__restrict__ vg, const int32_t *__restrict__ table_row,
    int32_t n, int32_t num_kv_heads, int32_t block_size, int32_t num_blocks, int32_t row_chunks) {
  const int64_t total = (int64_t)num_kv_heads * n * row_chunks;
  for (int64_t i = grid_stride_start(); i < total; i += grid_stride()) {
    const int32_t c = (int32_t)(i % row_chunks);
    const int64_t rest = i / row_chunks;
    const int32_t j = (int32_t)(rest % n);
    const int32_t g = (int32_t)(rest / n);
    int32_t blk = table_row[j / block_size];
    blk = blk < 0 ? 0 : (blk >= num_blocks ? num_blocks - 1 : blk);
    const int64_t src =
        (((int64_t)blk * num_kv_heads + g) * block_size + j % block_size) * row_chunks + c;
    kg[i] = k_cache[src];
    vg[i] = v_cache[src];
  }
}

// Row regrouping between the packed layout [q, Hq, row] (rows of one
// sequence) and the grouped layout [Hkv, q, G, row].  to_grouped = 1 reads
// packed and writes grouped (queries); 0 the reverse (outputs).
__global__ __launch_bounds__(kThreads) void unfused_regroup_kernel(
    const u32x4 *__restrict__ src, u32x4 *__restrict__ dst, int32_t q, int32_t num_heads,
    int32_t group, int32_t row_chunks, int32_t to_grouped) {
  const int64_t total = (int64_t)q * num_heads * row_chunks;
  for (int64_t i = grid_stride_start(); i < total; i += grid_stride()) {
    const int32_t c = (int32_t)(i % row_chunks);
    const int64_t rest = i / row_chunks;     // packed row: t * Hq + h
    const int32_t h = (int32_t)(rest % num_heads);
    const int32_t t = (int32_t)(rest / num_heads);
    const int32_t g = h / group, jh = h % group;
    const int64_t grouped = (((int64_t)g * q + t) * group + jh) * row_chunks + c;
    if (to_grouped) dst[grouped] = src[i];
    else dst[i] = src[grouped];
  }
}

__device__ __forceinline__ float wave_max(float v) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Causal row softmax.  Row r of S (fp32, leading dimension ld, a multiple
// of 8) belongs to grouped row c = r mod (q*G), i.e. new token t = c / G,
// which sees keys j < vis = prefix + t + 1.  The visible part of the row is
// read once into registers (CHUNKS float4 per thread, so rows up to
// 1024 * CHUNKS keys), reduced for the maximum and the normaliser, and the
// normalised weights are written as P (entries j >= vis are 0).
template <typename ST, int CHUNKS>
__global__ __launch_bounds__(kThreads) void unfused_softmax_kernel(
    const float *__restrict__ S, typename ST::storage *__restrict__ P, int32_t rows, int32_t n,
    int32_t ld, int32_t qg, int32_t group, int32_t prefix) {
  __shared__ float red[kThreads / 64];
  const int tid = threadIdx.x, wave = tid / 64, lane = tid % 64;
  const int32_t nchunks = (n + 3) / 4;
  for (int32_t r = blockIdx.x; r < rows; r += gridDim.x) {
    const int32_t t = (r % qg) / group;
    const int32_t vis = prefix + t + 1;
    const f32x4 *row = reinterpret_cast<const f32x4 *>(S + (int64_t)r * ld);
    f32x4 x[CHUNKS];
    float m = -INFINITY;
#pragma unroll
    for (int k = 0; k < CHUNKS; ++k) {
      const int32_t ci = tid + k * kThreads;
      x[k] = f32x4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
      if (ci * 4 < vis) {
        const f32x4 v = row[ci];
#pragma unroll
        for (int e = 0; e < 4; ++e) x[k][e] = (ci * 4 + e < vis) ? v[e] : -INFINITY;
      }
      m = fmaxf(m, fmaxf(fmaxf(x[k][0], x[k][1]), fmaxf(x[k][2], x[k][3])));
    }
    m = wave_max(m);
    if (lane == 0) red[wave] = m;
    __syncthreads();
    m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    __syncthreads();
    float l = 0.f;
#pragma unroll
    for (int k = 0; k < CHUNKS; ++k) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[k][e] = __expf(x[k][e] - m);     // masked: exp(-inf) = 0
        l += x[k][e];
      }
    }
    l = wave_sum(l);
    if (lane == 0) red[wave] = l;
    __syncthreads();
    const float inv = 1.0f / ((red[0] + red[1]) + (red[2] + red[3]));
    __syncthreads();
    u32x2 *prow = reinterpret_cast<u32x2 *>(P + (int64_t)r * ld);
#pragma unroll
    for (int k = 0; k < CHUNKS; ++k) {
      const int32_t ci = tid + k * kThreads;
      if (ci < nchunks) {
        const f32x4 p = x[k] * inv;
        if constexpr (std::is_same<ST, BF16>::value)
          prow[ci] = u32x2{pack_bf16(p[0], p[1]), pack_bf16(p[2], p[3])};
        else
          prow[ci] = u32x2{pack_f16(p[0], p[1]), pack_f16(p[2], p[3])};
      }
    }
  }
}

template <typename ST>
hipError_t launch_softmax(const float *S, void *P, int32_t rows, int32_t n, int32_t ld, int32_t qg,
                          int32_t group, int32_t prefix, hipStream_t stream) {
  typedef typename ST::storage E;
  const int grid = rows < 65536 ? rows : 65536;
  const int32_t per_thread = ((n + 3) / 4 + kThreads - 1) / kThreads;
#define PA_SOFTMAX(C)                                                                         \
  hipLaunchKernelGGL((unfused_softmax_kernel<ST, C>), dim3(grid), dim3(kThreads), 0, stream, S, \
                     static_cast<E *>(P), rows, n, ld, qg, group, prefix)
  if (per_thread <= 2) PA_SOFTMAX(2);
  else if (per_thread <= 4) PA_SOFTMAX(4);
  else if (per_thread <= 8) PA_SOFTMAX(8);
  else if (per_thread <= 16) PA_SOFTMAX(16);
  else if (per_thread <= 32) PA_SOFTMAX(32);
  else return hipErrorInvalidValue;
#undef PA_SOFTMAX
  return hipGetLastError();
}

// ---- hipBLASLt ------------------------------------------------------------

struct GemmShape {
  hipDataType ab, d;
  hipblasOperation_t ta;
  int64_t m, n, k, lda, ldb, ldd, sa, sb, sd;
  int32_t batch;
  auto key() const {
    return std::make_tuple((int)ab, (int)d, (int)ta, m, n, k, lda, ldb, ldd, sa, sb, sd, batch);
  }
  bool operator<(const GemmShape &o) const { return key() < o.key(); }
};

std::mutex g_blas_mu;
hipblasLtHandle_t g_handles[64] = {};
std::map<std::pair<int, GemmShape>, hipblasLtMatmulAlgo_t> g_algos;

hipblasLtHandle_t blas_handle(int dev) {
  std::lock_guard<std::mutex> lk(g_blas_mu);
  if (dev < 0 || dev >= 64) return nullptr;
  if (!g_handles[dev] && hipblasLtCreate(&g_handles[dev]) != HIPBLAS_STATUS_SUCCESS)
    g_handles[dev] = nullptr;
  return g_handles[dev];
}

struct Layouts {
  hipblasLtMatmulDesc_t desc = nullptr;
  hipblasLtMatrixLayout_t a = nullptr, b = nullptr, d = nullptr;
  ~Layouts() {
    if (a) hipblasLtMatrixLayoutDestroy(a);
    if (b) hipblasLtMatrixLayoutDestroy(b);
    if (d) hipblasLtMatrixLayoutDestroy(d);
    if (desc) hipblasLtMatmulDescDestroy(desc);
  }
};

bool make_layout(hipblasLtMatrixLayout_t *l, hipDataType t, int64_t rows, int64_t cols, int64_t ld,
                 int32_t batch, int64_t stride) {
  if (hipblasLtMatrixLayoutCreate(l, t, rows, cols, ld) != HIPBLAS_STATUS_SUCCESS) return false;
  return hipblasLtMatrixLayoutSetAttribute(*l, HIPBLASLT_MATRIX_LAYOUT_BATCH_COUNT, &batch,
                                           sizeof(batch)) == HIPBLAS_STATUS_SUCCESS &&
         hipblasLtMatrixLayoutSetAttribute(*l, HIPBLASLT_MATRIX_LAYOUT_STRIDED_BATCH_OFFSET,
                                           &stride, sizeof(stride)) == HIPBLAS_STATUS_SUCCESS;
}

// D = alpha * op(A) B over `batch` strided matrices (column-major, as the
// library counts): op(A) m x k, B k x n, D m x n (C = D with beta = 0).
pa_gemm_status run_gemm(int dev, const GemmShape &g, float alpha, const void *A, const void *B,
                        void *D, void *ws, size_t ws_bytes, hipStream_t stream) {
  hipblasLtHandle_t h = blas_handle(dev);
  if (!h) return PA_GEMM_NO_HANDLE;
  Layouts L;
  const hipblasOperation_t tn = HIPBLAS_OP_N;
  if (hipblasLtMatmulDescCreate(&L.desc, HIPBLAS_COMPUTE_32F, HIP_R_32F) != HIPBLAS_STATUS_SUCCESS ||
      hipblasLtMatmulDescSetAttribute(L.desc, HIPBLASLT_MATMUL_DESC_TRANSA, &g.ta, sizeof(g.ta)) !=
          HIPBLAS_STATUS_SUCCESS ||
      hipblasLtMatmulDescSetAttribute(L.desc, HIPBLASLT_MATMUL_DESC_TRANSB, &tn, sizeof(tn)) !=
          HIPBLAS_STATUS_SUCCESS)
    return PA_GEMM_UNSUPPORTED;
  const bool ta = g.ta == HIPBLAS_OP_T;
  if (!make_layout(&L.a, g.ab, ta ? g.k : g.m, ta ? g.m : g.k, g.lda, g.batch, g.sa) ||
      !make_layout(&L.b, g.ab, g.k, g.n, g.ldb, g.batch, g.sb) ||
      !make_layout(&L.d, g.d, g.m, g.n, g.ldd, g.batch, g.sd))
    return PA_GEMM_UNSUPPORTED;
  hipblasLtMatmulAlgo_t algo;
  {
    std::lock_guard<std::mutex> lk(g_blas_mu);
    auto it = g_algos.find({dev, g});
    if (it != g_algos.end()) {
      algo = it->second;
    } else {
      hipblasLtMatmulPreference_t pref = nullptr;
      const uint64_t max_ws = ws_bytes;
      hipblasLtMatmulHeuristicResult_t res[1];
      int found = 0;
      const bool ok =
          hipblasLtMatmulPreferenceCreate(&pref) == HIPBLAS_STATUS_SUCCESS &&
          hipblasLtMatmulPreferenceSetAttribute(pref, HIPBLASLT_MATMUL_PREF_MAX_WORKSPACE_BYTES,
                                                &max_ws, sizeof(max_ws)) ==
              HIPBLAS_STATUS_SUCCESS &&
          hipblasLtMatmulAlgoGetHeuristic(h, L.desc, L.a, L.b, L.d, L.d, pref, 1, res, &found) ==
              HIPBLAS_STATUS_SUCCESS &&
          found > 0 && res[0].workspaceSize <= ws_bytes;
      if (pref) hipblasLtMatmulPreferenceDestroy(pref);
      if (!ok) return PA_GEMM_UNSUPPORTED;
      algo = res[0].algo;
      g_algos.emplace(std::make_pair(dev, g), algo);
    }
  }
  const float beta = 0.0f;
  const hipblasStatus_t st = hipblasLtMatmul(h, L.desc, &alpha, A, L.a, B, L.b, &beta, D, L.d, D,
                                             L.d, &algo, ws, ws_bytes, stream);
  return st == HIPBLAS_STATUS_SUCCESS ? PA_GEMM_OK : PA_GEMM_FAILED;
}

inline size_t align_up(size_t v) { return (v + 255) & ~(size_t)255; }

}  // namespace

UnfusedWorkspace unfused_workspace_layout(int64_t max_q, int64_t max_ctx, int64_t num_heads,
                                          int64_t num_kv_heads, int64_t head_dim,
                                          int64_t elem_bytes) {
  UnfusedWorkspace w;
  const int64_t ld = (max_ctx + 7) / 8 * 8;
  size_t off = 0;
  w.kg_off = off;
  off += align_up((size_t)(num_kv_heads * max_ctx * head_dim * elem_bytes));
  w.vg_off = off;
  off += align_up((size_t)(num_kv_heads * max_ctx * head_dim * elem_bytes));
  w.qg_off = off;
  off += align_up((size_t)(max_q * num_heads * head_dim * elem_bytes));
  w.og_off = off;
  off += align_up((size_t)(max_q * num_heads * head_dim * elem_bytes));
  w.s_off = off;
  off += align_up((size_t)(num_heads * max_q * ld * 4));
  w.p_off = off;
  off += align_up((size_t)(num_heads * max_q * ld * elem_bytes));
  w.blas_off = off;
  w.blas_bytes = kUnfusedBlasWorkspace;
  off += kUnfusedBlasWorkspace;
  w.total = off;
  return w;
}

pa_gemm_status launch_prefill_unfused(const UnfusedLaunch &a, hipStream_t stream) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return PA_GEMM_FAILED;
  const int64_t e = a.dtype == DType::BF16 || a.dtype == DType::F16 ? 2 : 4;
  const hipDataType ab = a.dtype == DType::BF16 ? HIP_R_16BF : HIP_R_16F;
  const int32_t group = a.num_heads / a.num_kv_heads;
  const int32_t row_chunks = (int32_t)(a.head_dim * e / 16);
  const UnfusedWorkspace w = unfused_workspace_layout(a.max_q, a.max_ctx, a.num_heads,
                                                      a.num_kv_heads, a.head_dim, e);
  char *base = static_cast<char *>(a.workspace);
  u32x4 *kg = reinterpret_cast<u32x4 *>(base + w.kg_off);
  u32x4 *vg = reinterpret_cast<u32x4 *>(base + w.vg_off);
  u32x4 *qg = reinterpret_cast<u32x4 *>(base + w.qg_off);
  u32x4 *og = reinterpret_cast<u32x4 *>(base + w.og_off);
  float *S = reinterpret_cast<float *>(base + w.s_off);
  void *P = base + w.p_off;
  void *blas_ws = base + w.blas_off;
  const u32x4 *query = static_cast<const u32x4 *>(a.query);
  u32x4 *out = static_cast<u32x4 *>(a.out);
  const int64_t D = a.head_dim;

  for (int32_t b = 0; b < a.num_seqs; ++b) {
    const int32_t qs = a.query_start_loc[b];
    const int32_t q = a.query_start_loc[b + 1] - qs;
    const int32_t n = a.context_lens[b];
    if (q == 0) continue;
    const int32_t prefix = n - q;
    const int32_t ld = (n + 7) / 8 * 8;
    const int32_t qg_rows = q * group;
    auto grid_for = [](int64_t items) {
      const int64_t g = (items + kThreads - 1) / kThreads;
      return (unsigned)(g < 8192 ? (g > 0 ? g : 1) : 8192);
    };
    hipLaunchKernelGGL(unfused_gather_kv_kernel, dim3(grid_for((int64_t)a.num_kv_heads * n * row_chunks)),
                       dim3(kThreads), 0, stream, static_cast<const u32x4 *>(a.k_cache),
                       static_cast<const u32x4 *>(a.v_cache), kg, vg,
                       a.block_tables + (int64_t)b * a.max_blocks_per_seq, n, a.num_kv_heads,
                       a.block_size, a.num_blocks, row_chunks);
    hipLaunchKernelGGL(unfused_regroup_kernel, dim3(grid_for((int64_t)q * a.num_heads * row_chunks)),
                       dim3(kThreads), 0, stream, query + (int64_t)qs * a.num_heads * row_chunks, qg,
                       q, a.num_heads, group, row_chunks, 1);
    if (hipGetLastError() != hipSuccess) return PA_GEMM_FAILED;

    // S_g [n x q*G] (column-major) = scale * K_g Q_g^T: A = K_g stored
    // [D x n] (transposed), B = Q_g stored [D x q*G].
    GemmShape g1{ab, HIP_R_32F, HIPBLAS_OP_T, n, qg_rows, D, D, D, ld,
                 (int64_t)n * D, (int64_t)qg_rows * D, (int64_t)qg_rows * ld, a.num_kv_heads};
    pa_gemm_status st = run_gemm(dev, g1, a.scale, kg, qg, S, blas_ws, w.blas_bytes, stream);
    if (st != PA_GEMM_OK) return st;

    const hipError_t se =
        a.dtype == DType::BF16
            ? launch_softmax<BF16>(S, P, a.num_kv_heads * qg_rows, n, ld, qg_rows, group, prefix, stream)
            : launch_softmax<F16>(S, P, a.num_kv_heads * qg_rows, n, ld, qg_rows, group, prefix, stream);
    if (se != hipSuccess) return PA_GEMM_FAILED;

    // O_g^T [D x q*G] = V_g^T P_g^T: A = V_g stored [D x n], B = P_g stored
    // [n x q*G] with leading dimension ld.
    GemmShape g2{ab, ab, HIPBLAS_OP_N, D, qg_rows, n, D, ld, D,
                 (int64_t)n * D, (int64_t)qg_rows * ld, (int64_t)qg_rows * D, a.num_kv_heads};
    st = run_gemm(dev, g2, 1.0f, vg, P, og, blas_ws, w.blas_bytes, stream);
    if (st != PA_GEMM_OK) return st;

    hipLaunchKernelGGL(unfused_regroup_kernel, dim3(grid_for((int64_t)q * a.num_heads * row_chunks)),
                       dim3(kThreads), 0, stream, og, out + (int64_t)qs * a.num_heads * row_chunks,
                       q, a.num_heads, group, row_chunks, 0);
    if (hipGetLastError() != hipSuccess) return PA_GEMM_FAILED;
  }
  return PA_GEMM_OK;
}

}  // namespace pa
