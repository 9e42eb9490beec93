// The projections around the path ("Diffuser" reading notes, section 2.1,
// the per-head Q, K, V of the input and the head concatenation with the
// output projection outside the diffusion module, section 2.4):
//   [Q | K | V] = X W_qkv   (X: [B][n][d_model], W_qkv: [d_model][3 H d]),
//   Z = the whole path on (Q, K, V) per (b, h),
//   Y = concat_h(Z) W_o     (W_o: [H d][d_model], Y: [B][n][d_model]).
// Both products are plain dense GEMMs (rocBLAS, fp32 accumulation); the
// head split and merge are elementwise kernels of 16-byte chunks.
#include <rocblas/rocblas.h>

#include <mutex>

#include "internal.h"
#include "vec.h"

namespace diffuser {
namespace {

constexpr int kThreads = 256;

// out[p][b][h][i][c] = T[b n + i][p H d + h d + c] for p = 0, 1, 2, in
// chunks of E elements (one 16-byte chunk per thread).
template <typename T>
__global__ __launch_bounds__(kThreads)
void k_split_heads(int64_t rows, int32_t n, int32_t H, int32_t d, const T* __restrict__ in,
                   T* __restrict__ q, T* __restrict__ k, T* __restrict__ v) {
    constexpr int E = chunk<T>::kElems;
    const int32_t per_row = 3 * H * d / E;
    const int64_t total = rows * per_row;
    for (int64_t t = (int64_t)blockIdx.x * kThreads + threadIdx.x; t < total;
         t += (int64_t)gridDim.x * kThreads) {
        const int64_t r = t / per_row;
        const int32_t col = (int32_t)(t - r * per_row) * E;
        const int32_t p = col / (H * d), hc = col - p * H * d, h = hc / d, c = hc - h * d;
        const int64_t b = r / n, i = r - b * n;
        T* dst = p == 0 ? q : (p == 1 ? k : v);
        *reinterpret_cast<uint4*>(dst + (((b * H + h) * n + i) * d + c)) =
            *reinterpret_cast<const uint4*>(in + r * 3 * H * d + col);
    }
}

// out[b n + i][h d + c] = Z[b][h][i][c].
template <typename T>
__global__ __launch_bounds__(kThreads)
void k_merge_heads(int64_t rows, int32_t n, int32_t H, int32_t d, const T* __restrict__ z,
                   T* __restrict__ out) {
    constexpr int E = chunk<T>::kElems;
    const int32_t per_row = H * d / E;
    const int64_t total = rows * per_row;
    for (int64_t t = (int64_t)blockIdx.x * kThreads + threadIdx.x; t < total;
         t += (int64_t)gridDim.x * kThreads) {
        const int64_t r = t / per_row;
        const int32_t col = (int32_t)(t - r * per_row) * E;
        const int32_t h = col / d, c = col - h * d;
        const int64_t b = r / n, i = r - b * n;
        *reinterpret_cast<uint4*>(out + r * H * d + col) =
            *reinterpret_cast<const uint4*>(z + (((b * H + h) * n + i) * d + c));
    }
}

dim3 grid_for(int64_t work) {
    int64_t blocks = (work + kThreads - 1) / kThreads;
    if (blocks > 65536) blocks = 65536;
    return dim3((unsigned)(blocks < 1 ? 1 : blocks));
}

// One rocBLAS handle per device, created on first use; calls that share it
// are serialised (the stream and workspace are set per call).
struct BlasHandles {
    std::mutex mu;
    rocblas_handle h[64] = {};
};

BlasHandles& blas_handles() {
    static BlasHandles hs;
    return hs;
}

// Row-major C[M][N] = A[M][K] B[K][N] (column-major C^T = B^T A^T).
rocblas_status gemm_rm(rocblas_handle h, diffuser_dtype t, int64_t M, int64_t N, int64_t K,
                       const void* A, const void* B, void* C) {
    const float one = 1.0f, zero = 0.0f;
    const rocblas_datatype dt = t == DIFFUSER_F32 ? rocblas_datatype_f32_r : rocblas_datatype_bf16_r;
    return rocblas_gemm_ex_64(h, rocblas_operation_none, rocblas_operation_none, N, M, K, &one, B,
                              dt, N, A, dt, K, &zero, C, dt, N, C, dt, N, rocblas_datatype_f32_r,
                              rocblas_gemm_algo_standard, 0, 0);
}

}  // namespace

hipError_t launch_split_heads(diffuser_dtype t, int64_t B, int32_t n, int32_t H, int32_t d,
                              const void* in, void* q, void* k, void* v, hipStream_t st) {
    const int64_t rows = B * n;
    if (t == DIFFUSER_F32)
        hipLaunchKernelGGL(k_split_heads<float>, grid_for(rows * 3 * H * d / 4), dim3(kThreads),
                           0, st, rows, n, H, d, static_cast<const float*>(in),
                           static_cast<float*>(q), static_cast<float*>(k), static_cast<float*>(v));
    else
        hipLaunchKernelGGL(k_split_heads<bf16_t>, grid_for(rows * 3 * H * d / 8), dim3(kThreads),
                           0, st, rows, n, H, d, static_cast<const bf16_t*>(in),
                           static_cast<bf16_t*>(q), static_cast<bf16_t*>(k),
                           static_cast<bf16_t*>(v));
    return hipGetLastError();
}

hipError_t launch_merge_heads(diffuser_dtype t, int64_t B, int32_t n, int32_t H, int32_t d,
                              const void* z, void* out, hipStream_t st) {
    const int64_t rows = B * n;
    if (t == DIFFUSER_F32)
        hipLaunchKernelGGL(k_merge_heads<float>, grid_for(rows * H * d / 4), dim3(kThreads), 0, st,
                           rows, n, H, d, static_cast<const float*>(z), static_cast<float*>(out));
    else
        hipLaunchKernelGGL(k_merge_heads<bf16_t>, grid_for(rows * H * d / 8), dim3(kThreads), 0,
                           st, rows, n, H, d, static_cast<const bf16_t*>(z),
                           static_cast<bf16_t*>(out));
    return hipGetLastError();
}

diffuser_status blas_gemm(int device, diffuser_dtype t, int64_t M, int64_t N, int64_t K,
                          const void* A, const void* B, void* C, void* blas_ws,
                          size_t blas_ws_bytes, hipStream_t st) {
    BlasHandles& hs = blas_handles();
    std::lock_guard<std::mutex> lock(hs.mu);
    if (device < 0 || device >= 64) return fail(DIFFUSER_ERR_UNSUPPORTED, "device index >= 64");
    if (hs.h[device] == nullptr && rocblas_create_handle(&hs.h[device]) != rocblas_status_success)
        return fail(DIFFUSER_ERR_INTERNAL, "rocblas_create_handle failed");
    rocblas_handle h = hs.h[device];
    if (rocblas_set_stream(h, st) != rocblas_status_success ||
        rocblas_set_workspace(h, blas_ws, blas_ws_bytes) != rocblas_status_success)
        return fail(DIFFUSER_ERR_INTERNAL, "rocblas stream/workspace setup failed");
    const rocblas_status s = gemm_rm(h, t, M, N, K, A, B, C);
    rocblas_set_workspace(h, nullptr, 0);
    if (s != rocblas_status_success)
        return fail(DIFFUSER_ERR_INTERNAL, std::string("rocblas_gemm_ex: ") +
                                               rocblas_status_to_string(s));
    return DIFFUSER_OK;
}

}  // namespace diffuser
