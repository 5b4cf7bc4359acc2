// Joint-ITQ rotation on the device ([LB2 column] Ch. 2): an orthogonal R
// between the factors leaves U V^T unchanged, so the factors may be rotated
// before binarising; R is found by iterative quantisation of the stacked
// factors X = [U; V] ((b + a) x s).  A step quantises, B = sign(X R) with
// sign(0) = +1, then takes the rotation that best maps X onto B, the
// orthogonal polar factor of M = X^T B (the orthogonal Procrustes
// solution).
//
// Everything is fp64 (X is converted once from the fp32 factors).  The
// three products of a step are plain dense GEMMs and go to rocBLAS dgemm
// (atomics off, so results are reproducible):
//   Y = X R      ((b + a) x s) x (s x s), then B = sign(Y) in place
//   M = X^T B    a reduction over the b + a rows, split into up to 32 row
//                chunks (one strided-batched dgemm) summed in a fixed order
//   polar(M)     Newton-Schulz: Z0 = M / ||M||_F (every singular value in
//                (0, 1]), Z <- Z (3 I - Z^T Z) / 2, two s x s x s products
//                per step, until max |Z^T Z - I| <= 1e-12; it converges to
//                the orthogonal polar factor whenever M is nonsingular.
// Matrices are row-major; a row-major matrix is the column-major transpose,
// so C = A B row-major is dgemm(N, N) on (B, A).
#include <hip/hip_runtime.h>
#include <rocblas/rocblas.h>
#include <stdint.h>

#include <algorithm>
#include <cmath>
#include <map>
#include <mutex>
#include <string>

#include "lb_internal.h"

namespace lbi {
namespace {

constexpr int kNsMaxSteps = 200;
constexpr int kNsCheckEvery = 3;
constexpr int kXtbChunks = 32;
constexpr double kNsTol = 1e-12;

__global__ void __launch_bounds__(256) k_stack_f64(const float *__restrict__ U,
                                                   const float *__restrict__ V, int64_t nu,
                                                   int64_t total, double *__restrict__ X) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * 256)
    X[i] = i < nu ? (double)U[i] : (double)V[i - nu];
}

__global__ void __launch_bounds__(256) k_sign_pm1(double *__restrict__ Y, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    Y[i] = Y[i] >= 0.0 ? 1.0 : -1.0;
}

__global__ void __launch_bounds__(256) k_eye(double *__restrict__ R, int64_t s) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < s * s;
       i += (int64_t)gridDim.x * 256)
    R[i] = (i / s == i % s) ? 1.0 : 0.0;
}

__global__ void __launch_bounds__(256) k_copy_f64(const double *__restrict__ a,
                                                  double *__restrict__ b, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    b[i] = a[i];
}

// out[k] = sum over c of part[c][k] (nc partial s x s products, in order).
__global__ void __launch_bounds__(256) k_sum_parts(const double *__restrict__ part, int nc,
                                                   int64_t n, double *__restrict__ out) {
  for (int64_t k = (int64_t)blockIdx.x * 256 + threadIdx.x; k < n; k += (int64_t)gridDim.x * 256) {
    double acc = 0.0;
    for (int c = 0; c < nc; ++c) acc += part[(size_t)c * n + k];
    out[k] = acc;
  }
}

// Block partials over an s x s matrix (nb blocks, each a contiguous range
// of rows; a wave per row, lanes along the row):
//   k_sq_parts:  part[blk] = sum of squares, in a fixed order
//   k_err_parts: part[blk] = max |T - I|
constexpr int kNsBlocks = 64;

__device__ inline void row_range(int64_t s, int64_t *r0, int64_t *r1) {
  const int64_t per = (s + gridDim.x - 1) / gridDim.x;
  *r0 = (int64_t)blockIdx.x * per;
  *r1 = (*r0 + per) < s ? (*r0 + per) : s;
}

__global__ void __launch_bounds__(256) k_sq_parts(const double *__restrict__ M, int64_t s,
                                                  double *__restrict__ part) {
  __shared__ double sh[256];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  int64_t r0, r1;
  row_range(s, &r0, &r1);
  double acc = 0.0;
  for (int64_t r = r0 + wave; r < r1; r += 4)
    for (int64_t c = lane; c < s; c += 64) acc += M[(size_t)r * s + c] * M[(size_t)r * s + c];
  sh[t] = acc;
  __syncthreads();
  for (int o = 128; o >= 1; o >>= 1) {
    if (t < o) sh[t] += sh[t + o];
    __syncthreads();
  }
  if (t == 0) part[blockIdx.x] = sh[0];
}

__global__ void __launch_bounds__(256) k_err_parts(const double *__restrict__ T, int64_t s,
                                                   double *__restrict__ part) {
  __shared__ double sh[256];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  int64_t r0, r1;
  row_range(s, &r0, &r1);
  double m = 0.0;
  for (int64_t r = r0 + wave; r < r1; r += 4)
    for (int64_t c = lane; c < s; c += 64)
      m = fmax(m, fabs(T[(size_t)r * s + c] - (c == r ? 1.0 : 0.0)));
  sh[t] = m;
  __syncthreads();
  for (int o = 128; o >= 1; o >>= 1) {
    if (t < o) sh[t] = fmax(sh[t], sh[t + o]);
    __syncthreads();
  }
  if (t == 0) part[blockIdx.x] = sh[0];
}

// Z = M / ||M||_F and C = Z; every thread adds the nb partials in the same
// order, so all blocks use the same norm.
__global__ void __launch_bounds__(256) k_ns_scale(const double *__restrict__ M, int64_t n,
                                                  const double *__restrict__ part, int nb,
                                                  double *__restrict__ Z,
                                                  double *__restrict__ C) {
  double ss = 0.0;
  for (int i = 0; i < nb; ++i) ss += part[i];
  const double nrm = sqrt(ss);
  const double inv = nrm > 0.0 ? 1.0 / nrm : 0.0;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    const double z = M[i] * inv;
    Z[i] = z;
    C[i] = z;
  }
}

inline unsigned grid_of(int64_t n, int per, int64_t cap = 65536) {
  const int64_t g = (n + per - 1) / per;
  return (unsigned)(g < cap ? g : cap);
}

// rocBLAS handles, one per device, created on first use.  A mutex
// serialises the calls that use them (initialisation is a setup step).
std::mutex g_blas_mu;
std::map<int, rocblas_handle> g_blas;

int blas_for(int device, rocblas_handle *out, std::string *msg) {
  auto it = g_blas.find(device);
  if (it == g_blas.end()) {
    rocblas_handle h = nullptr;
    if (rocblas_create_handle(&h) != rocblas_status_success) {
      *msg = "rocblas_create_handle failed";
      return LB_EHIP;
    }
    if (rocblas_set_atomics_mode(h, rocblas_atomics_not_allowed) != rocblas_status_success) {
      *msg = "rocblas_set_atomics_mode failed";
      return LB_EHIP;
    }
    it = g_blas.emplace(device, h).first;
  }
  *out = it->second;
  return 0;
}

// Row-major C (m x n) = alpha A (m x k) B (k x n) + beta C, with op flags on
// the row-major operands (trans_a: A is stored k x m).
int gemm_rm(rocblas_handle h, bool trans_a, bool trans_b, int64_t m, int64_t n, int64_t k,
            double alpha, const double *A, const double *B, double beta, double *C,
            std::string *msg) {
  // column-major: C^T (n x m) = op(B)^T op(A)^T
  const rocblas_operation ob = trans_b ? rocblas_operation_transpose : rocblas_operation_none;
  const rocblas_operation oa = trans_a ? rocblas_operation_transpose : rocblas_operation_none;
  const rocblas_int ldb = (rocblas_int)(trans_b ? k : n);
  const rocblas_int lda = (rocblas_int)(trans_a ? m : k);
  const rocblas_status st = rocblas_dgemm(h, ob, oa, (rocblas_int)n, (rocblas_int)m,
                                          (rocblas_int)k, &alpha, B, ldb, A, lda, &beta, C,
                                          (rocblas_int)n);
  if (st != rocblas_status_success) {
    *msg = std::string("rocblas_dgemm: ") + rocblas_status_to_string(st);
    return LB_EHIP;
  }
  return 0;
}

// Row-major M (s x s) = X^T Y over n rows, split into nc row chunks of L
// rows (the last may be shorter): the chunk products M_c = X_c^T Y_c go to
// part[c] (one strided-batched dgemm for the full chunks), then a fixed-order
// sum.  A single dgemm would give only a few output tiles the whole
// reduction (its split-K needs atomics, which are off).
int xtb_split(rocblas_handle h, const double *X, const double *Y, int64_t n, int64_t s, int nc,
              double *part, double *M, hipStream_t st, std::string *msg) {
  const int64_t L = (n + nc - 1) / nc;
  const int64_t nfull = n / L, rem = n - nfull * L;
  const double one = 1.0, zero = 0.0;
  if (nfull > 0) {
    // gemm_rm(trans_a = true) on (X_c, Y_c), batched over the chunks
    const rocblas_status stt = rocblas_dgemm_strided_batched(
        h, rocblas_operation_none, rocblas_operation_transpose, (rocblas_int)s, (rocblas_int)s,
        (rocblas_int)L, &one, Y, (rocblas_int)s, (rocblas_stride)(L * s), X, (rocblas_int)s,
        (rocblas_stride)(L * s), &zero, part, (rocblas_int)s, (rocblas_stride)(s * s),
        (rocblas_int)nfull);
    if (stt != rocblas_status_success) {
      *msg = std::string("rocblas_dgemm_strided_batched: ") + rocblas_status_to_string(stt);
      return LB_EHIP;
    }
  }
  if (rem > 0) {
    const int rc = gemm_rm(h, true, false, s, s, rem, 1.0, X + (size_t)nfull * L * s,
                           Y + (size_t)nfull * L * s, 0.0, part + (size_t)nfull * s * s, msg);
    if (rc != 0) return rc;
  }
  const int parts = (int)(nfull + (rem > 0 ? 1 : 0));
  hipLaunchKernelGGL(k_sum_parts, dim3(grid_of(s * s, 256)), dim3(256), 0, st, part, parts, s * s,
                     M);
  if (hipGetLastError() != hipSuccess) {
    *msg = "k_sum_parts launch";
    return LB_EHIP;
  }
  return 0;
}

#define ITQ_HIP(call)                                                     \
  do {                                                                    \
    hipError_t e_ = (call);                                               \
    if (e_ != hipSuccess) {                                               \
      *msg = std::string(#call) + ": " + hipGetErrorString(e_);           \
      return LB_EHIP;                                                     \
    }                                                                     \
  } while (0)

#define ITQ_TRY(expr)        \
  do {                       \
    const int r_ = (expr);   \
    if (r_ != 0) return r_;  \
  } while (0)

// Orthogonal polar factor of M (s x s) into R by Newton-Schulz; Z, C, T are
// s x s scratch and part holds kNsBlocks doubles.  Convergence is checked
// every kNsCheckEvery steps from step *first_check on (the previous call's
// step count less a margin: successive M of one Joint-ITQ run are alike),
// and *first_check is updated.  Returns LB_EUNSUPPORTED when it does not
// settle (M singular or nearly so).
int polar_ns(rocblas_handle h, const double *M, int64_t s, double *R, double *Z, double *C,
             double *T, double *part, int *first_check, hipStream_t st, std::string *msg) {
  const int64_t n = s * s;
  const int nb = (int)std::min<int64_t>(kNsBlocks, s);
  hipLaunchKernelGGL(k_sq_parts, dim3(nb), dim3(256), 0, st, M, s, part);
  hipLaunchKernelGGL(k_ns_scale, dim3(grid_of(n, 256, 512)), dim3(256), 0, st, M, n, part, nb, Z,
                     C);
  ITQ_HIP(hipGetLastError());
  double err[kNsBlocks];
  for (int step = 0; step < kNsMaxSteps; ++step) {
    ITQ_TRY(gemm_rm(h, true, false, s, s, s, 1.0, Z, Z, 0.0, T, msg));  // T = Z^T Z
    if (step >= *first_check && (step - *first_check) % kNsCheckEvery == 0) {
      hipLaunchKernelGGL(k_err_parts, dim3(nb), dim3(256), 0, st, T, s, part);
      ITQ_HIP(hipGetLastError());
      ITQ_HIP(hipMemcpyAsync(err, part, nb * sizeof(double), hipMemcpyDeviceToHost, st));
      ITQ_HIP(hipStreamSynchronize(st));
      double e = 0.0;
      for (int i = 0; i < nb; ++i) e = e > err[i] ? e : err[i];
      if (e <= kNsTol) {
        hipLaunchKernelGGL(k_copy_f64, dim3(grid_of(n, 256)), dim3(256), 0, st, Z, R, n);
        ITQ_HIP(hipGetLastError());
        *first_check = step > 4 ? step - 4 : 0;
        return 0;
      }
    }
    // C (= Z) <- 1.5 Z - 0.5 Z T, then Z <- C
    ITQ_TRY(gemm_rm(h, false, false, s, s, s, -0.5, Z, T, 1.5, C, msg));
    hipLaunchKernelGGL(k_copy_f64, dim3(grid_of(n, 256)), dim3(256), 0, st, C, Z, n);
    ITQ_HIP(hipGetLastError());
  }
  *msg = "Joint-ITQ: the polar factor of X^T B did not settle (X^T B singular or nearly so)";
  return LB_EUNSUPPORTED;
}

struct DevBuf {
  void *p = nullptr;
  ~DevBuf() {
    if (p) (void)hipFree(p);
  }
};

}  // namespace

int joint_itq_dev(const float *U, const float *V, int64_t a, int64_t b, int64_t s, int iters,
                  const double *R0, double *R, hipStream_t st, std::string *msg) {
  std::lock_guard<std::mutex> lk(g_blas_mu);
  int device = 0;
  ITQ_HIP(hipGetDevice(&device));
  rocblas_handle h = nullptr;
  ITQ_TRY(blas_for(device, &h, msg));
  if (rocblas_set_stream(h, st) != rocblas_status_success) {
    *msg = "rocblas_set_stream failed";
    return LB_EHIP;
  }
  const int64_t n = a + b, ss = s * s;
  // row chunks of X^T B: about 256 rows each, at most kXtbChunks
  const int nc = (int)std::min<int64_t>(kXtbChunks, (n + 255) / 256);
  // X (n x s), Y (n x s), M, Rw, Z, C, T (s x s), err (kNsBlocks), part (nc x s x s)
  DevBuf buf;
  const size_t doubles = (size_t)2 * n * s + 5 * (size_t)ss + kNsBlocks + (size_t)nc * ss;
  if (hipMalloc(&buf.p, doubles * sizeof(double)) != hipSuccess) {
    *msg = "Joint-ITQ: device allocation";
    return LB_ENOMEM;
  }
  double *X = static_cast<double *>(buf.p), *Y = X + (size_t)n * s, *M = Y + (size_t)n * s;
  double *Rw = M + ss, *Z = Rw + ss, *C = Z + ss, *T = C + ss, *err = T + ss;
  double *part = err + kNsBlocks;
  hipLaunchKernelGGL(k_stack_f64, dim3(grid_of(n * s, 256)), dim3(256), 0, st, U, V, b * s, n * s,
                     X);
  if (R0)
    hipLaunchKernelGGL(k_copy_f64, dim3(grid_of(ss, 256)), dim3(256), 0, st, R0, Rw, ss);
  else
    hipLaunchKernelGGL(k_eye, dim3(grid_of(ss, 256)), dim3(256), 0, st, Rw, s);
  ITQ_HIP(hipGetLastError());
  int first_check = 0;
  for (int it = 0; it < iters; ++it) {
    ITQ_TRY(gemm_rm(h, false, false, n, s, s, 1.0, X, Rw, 0.0, Y, msg));  // Y = X R
    hipLaunchKernelGGL(k_sign_pm1, dim3(grid_of(n * s, 256)), dim3(256), 0, st, Y, n * s);
    ITQ_HIP(hipGetLastError());
    ITQ_TRY(xtb_split(h, X, Y, n, s, nc, part, M, st, msg));  // M = X^T B
    ITQ_TRY(polar_ns(h, M, s, Rw, Z, C, T, err, &first_check, st, msg));
  }
  hipLaunchKernelGGL(k_copy_f64, dim3(grid_of(ss, 256)), dim3(256), 0, st, Rw, R, ss);
  ITQ_HIP(hipGetLastError());
  ITQ_HIP(hipStreamSynchronize(st));
  return 0;
}

int rotate_factors_dev(const float *U, const float *V, int64_t a, int64_t b, int64_t s,
                       const double *R, double *out, hipStream_t st, std::string *msg) {
  std::lock_guard<std::mutex> lk(g_blas_mu);
  int device = 0;
  ITQ_HIP(hipGetDevice(&device));
  rocblas_handle h = nullptr;
  ITQ_TRY(blas_for(device, &h, msg));
  if (rocblas_set_stream(h, st) != rocblas_status_success) {
    *msg = "rocblas_set_stream failed";
    return LB_EHIP;
  }
  const int64_t n = a + b;
  DevBuf buf;
  if (hipMalloc(&buf.p, (size_t)n * s * sizeof(double)) != hipSuccess) {
    *msg = "rotate factors: device allocation";
    return LB_ENOMEM;
  }
  double *X = static_cast<double *>(buf.p);
  hipLaunchKernelGGL(k_stack_f64, dim3(grid_of(n * s, 256)), dim3(256), 0, st, U, V, b * s, n * s,
                     X);
  ITQ_HIP(hipGetLastError());
  ITQ_TRY(gemm_rm(h, false, false, n, s, s, 1.0, X, R, 0.0, out, msg));
  ITQ_HIP(hipStreamSynchronize(st));  // X is freed on return
  return 0;
}

}  // namespace lbi
