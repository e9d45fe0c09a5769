// bluestein.hip -- element-wise kernels of the chirp-z (Bluestein) route to a
// transform of any length N, which "FFT on GPU" (section "Algorithm per
// signal Length") lists for lengths that are not powers of two.
//
// With c_j = e^{-i pi j^2 / N} and n k = (n^2 + k^2 - (k - n)^2) / 2,
//     X_k = c_k sum_n (x_n c_n) conj(c_{k-n}),
// a linear convolution, evaluated as a cyclic one of power-of-two length
// M >= 2N - 1 with the library's own power-of-two transforms:
//     w = pad_M(x . c);  W = F_M(w) . B;  y = F_M^{-1}(W);  X_k = c_k y_k,
// where B = F_M(b), b_m = conj(c_m) for m < N, b_{M-m} = conj(c_m) for
// 0 < m < N (computed once, in fp64, when the plan is made).
#include "io.hpp"
#include "launch.hpp"
#include "stockham.hpp"

namespace fftmi {

static inline dim3 ew_grid(int64_t total)
{
    int64_t blocks = (total + 255) / 256;
    if (blocks > (1 << 20)) blocks = 1 << 20;  // grid-stride beyond this
    return dim3((unsigned)(blocks > 0 ? blocks : 1));
}

// w[row][j] = x[row][j] c_j for j < n, 0 for n <= j < 2^logm.
template <typename V, bool PIN>
__global__ void chirp_pre_kernel(CIn<V, PIN> in, V* w, int64_t n, int logm, int64_t total,
                                 const V* __restrict__ chirp, int conj_in)
{
    const int64_t m_mask = ((int64_t)1 << logm) - 1;
    for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total; e += (int64_t)gridDim.x * blockDim.x) {
        const int64_t row = e >> logm, j = e & m_mask;
        V v{0, 0};
        if (j < n) {
            V x = in.ld_plain(row * n + j);
            if (conj_in) x = cconj(x);
            v = cmul(x, chirp[j]);
        }
        w[e] = v;
    }
}

// w[row][j] *= tab[j].
template <typename V>
__global__ void cmul_table_kernel(V* w, int logm, int64_t total, const V* __restrict__ tab)
{
    const int64_t m_mask = ((int64_t)1 << logm) - 1;
    for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total; e += (int64_t)gridDim.x * blockDim.x)
        w[e] = cmul(w[e], tab[e & m_mask]);
}

// out[row][k] = c_k y[row][k] for k < n (conjugated and scaled for the inverse).
template <typename V, bool POUT>
__global__ void chirp_post_kernel(const V* w, COut<V, POUT> out, int64_t n, int logm, int64_t total,
                                  const V* __restrict__ chirp, int conj_out, typename real_of<V>::type scale)
{
    for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total; e += (int64_t)gridDim.x * blockDim.x) {
        const int64_t row = e / n, k = e - row * n;
        const V y = cmul(w[(row << logm) + k], chirp[k]);
        out.st_plain(e, conj_out ? V{y.x * scale, -y.y * scale} : y);
    }
}

__global__ void narrow_kernel(const double2* __restrict__ in, float2* __restrict__ out, int64_t total)
{
    for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total; e += (int64_t)gridDim.x * blockDim.x)
        out[e] = float2{(float)in[e].x, (float)in[e].y};
}

template <typename V, bool PIN>
static void chirp_pre_t(const void* in, const void* in_im, void* w, int64_t n, int logm, int64_t total,
                        const void* chirp, bool conj_in, hipStream_t s)
{
    hipLaunchKernelGGL((chirp_pre_kernel<V, PIN>), ew_grid(total), dim3(256), 0, s, make_in<V, PIN>(in, in_im),
                       (V*)w, n, logm, total, (const V*)chirp, (int)conj_in);
}

hipError_t launch_chirp_pre(int prec, const void* in, void* w, int64_t n, int logm, int64_t batch, const void* chirp,
                            bool conj_in, hipStream_t s, const void* in_im)
{
    const int64_t total = batch << logm;
    if (prec == 0) {
        if (in_im) chirp_pre_t<float2, true>(in, in_im, w, n, logm, total, chirp, conj_in, s);
        else chirp_pre_t<float2, false>(in, in_im, w, n, logm, total, chirp, conj_in, s);
    } else {
        if (in_im) chirp_pre_t<double2, true>(in, in_im, w, n, logm, total, chirp, conj_in, s);
        else chirp_pre_t<double2, false>(in, in_im, w, n, logm, total, chirp, conj_in, s);
    }
    return hipGetLastError();
}

hipError_t launch_cmul_table(int prec, void* w, int logm, int64_t batch, const void* tab, hipStream_t s)
{
    const int64_t total = batch << logm;
    if (prec == 0)
        hipLaunchKernelGGL(cmul_table_kernel<float2>, ew_grid(total), dim3(256), 0, s, (float2*)w, logm, total,
                           (const float2*)tab);
    else
        hipLaunchKernelGGL(cmul_table_kernel<double2>, ew_grid(total), dim3(256), 0, s, (double2*)w, logm, total,
                           (const double2*)tab);
    return hipGetLastError();
}

template <typename V, bool POUT>
static void chirp_post_t(const void* w, void* out, void* out_im, int64_t n, int logm, int64_t total,
                         const void* chirp, bool conj_out, double scale, hipStream_t s)
{
    using Rl = typename real_of<V>::type;
    hipLaunchKernelGGL((chirp_post_kernel<V, POUT>), ew_grid(total), dim3(256), 0, s, (const V*)w,
                       make_out<V, POUT>(out, out_im), n, logm, total, (const V*)chirp, (int)conj_out, (Rl)scale);
}

hipError_t launch_chirp_post(int prec, const void* w, void* out, int64_t n, int logm, int64_t batch,
                             const void* chirp, bool conj_out, double scale, hipStream_t s, void* out_im)
{
    const int64_t total = batch * n;
    if (prec == 0) {
        if (out_im) chirp_post_t<float2, true>(w, out, out_im, n, logm, total, chirp, conj_out, scale, s);
        else chirp_post_t<float2, false>(w, out, out_im, n, logm, total, chirp, conj_out, scale, s);
    } else {
        if (out_im) chirp_post_t<double2, true>(w, out, out_im, n, logm, total, chirp, conj_out, scale, s);
        else chirp_post_t<double2, false>(w, out, out_im, n, logm, total, chirp, conj_out, scale, s);
    }
    return hipGetLastError();
}

hipError_t launch_narrow(const void* in, void* out, int64_t total, hipStream_t s)
{
    hipLaunchKernelGGL(narrow_kernel, ew_grid(total), dim3(256), 0, s, (const double2*)in, (float2*)out, total);
    return hipGetLastError();
}

}  // namespace fftmi
