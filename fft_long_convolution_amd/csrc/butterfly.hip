// butterfly.hip -- matrix images of caller-supplied (learned) factor blocks for the fused 1D
// kernels' learned-Butterfly mode.
//
// The "Simple Hardware-Efficient Long Convolutions for Sequence Modeling" abstract says the
// coefficients of the Butterfly decomposition can be learned.  Here the decomposition is the
// one the fused kernels run (n = 256 n1 + 16 n2 + n3, f = k1 + R k2 + 16 R k3): its dense
// factor blocks, which for the DFT are
//     A1[k1][n1] = w_R^{n1 k1}                    B3[n1][k1]     = conj A1[k1][n1]
//     A2[k1][k2][n2] = w_{16R}^{n2 (k1 + R k2)}   B2[k1][n2][k2] = conj A2[k1][k2][n2]
//     A3[k1][k3][n3] = w_M^{n3 (k1 + 16 R k3)}    B1[k1][n3][k3] = conj A3[k1][k3][n3]
// come from the caller instead; the twiddle w_256^{n3 k2} between the second and third stage
// stays fixed.  This kernel writes them in the lane layout the kernels load (the layout of the
// plan's own tables, plan.cpp), in fp32 and in the 16-bit compute type.
#include <hip/hip_runtime.h>

#include "kernels.h"
#include "lconv_device.h"

namespace lcv {

namespace {

struct BflyImgArgs {
    const float2* blocks;   // A1, A2, A3, B1, B2, B3 (fp32 complex)
    void* out;              // table in the fused layout for (R, ct)
    int R, ct;
    int rb;                 // F1 / I3 image grid side: (R + 15) / 16
    size_t f1, i3, f2, f3, i1, i2;  // byte offsets of the image groups
};

// G(x, ci) of image `img`: x = output index (lane % 16), ci = contracted index
__device__ float2 block_entry(const BflyImgArgs& a, int img, int x, int ci) {
    const int R = a.R, nf1 = a.rb * a.rb;
    const float2* A1 = a.blocks;
    const float2* A2 = A1 + R * R;
    const float2* A3 = A2 + R * 256;
    const float2* B1 = A3 + R * 256;
    const float2* B2 = B1 + R * 256;
    const float2* B3 = B2 + R * 256;
    const float2 zero = make_float2(0.f, 0.f);
    if (img < nf1) {  // F1 (rb, kc): rows k1 = 16 rb + x, inputs n1 = 16 kc + ci
        const int k1 = 16 * (img / a.rb) + x, n1 = 16 * (img % a.rb) + ci;
        return k1 < R && n1 < R ? A1[k1 * R + n1] : zero;
    }
    img -= nf1;
    if (img < nf1) {  // I3 (rb, kc): rows n1 = 16 rb + x, inputs k1 = 16 kc + ci
        const int n1 = 16 * (img / a.rb) + x, k1 = 16 * (img % a.rb) + ci;
        return k1 < R && n1 < R ? B3[n1 * R + k1] : zero;
    }
    img -= nf1;
    const int grp = img / R, k1 = img % R;
    const float2* src = grp == 0 ? A2 : grp == 1 ? A3 : grp == 2 ? B1 : B2;
    return src[k1 * 256 + x * 16 + ci];  // [k1][output][contracted]
}

__global__ void __launch_bounds__(64) bfly_images_kernel(const BflyImgArgs a) {
    const int img = blockIdx.x, lane = threadIdx.x, g = lane / 16, x = lane % 16;
    const int nf1 = a.rb * a.rb;
    size_t off;
    if (img < nf1) off = a.f1 + (size_t)img * (a.ct == CT_F32 ? 4096 : 2048);
    else if (img < 2 * nf1) off = a.i3 + (size_t)(img - nf1) * (a.ct == CT_F32 ? 4096 : 2048);
    else {
        const int i = img - 2 * nf1, grp = i / a.R, k1 = i % a.R;
        const size_t base = grp == 0 ? a.f2 : grp == 1 ? a.f3 : grp == 2 ? a.i1 : a.i2;
        off = base + (size_t)k1 * (a.ct == CT_F32 ? 4096 : 2048);
    }
    // slot s of the real-output operand: [Gr, -Gi]; of the imaginary-output one: [Gi, Gr]
    float v[16];
#pragma unroll
    for (int s = 0; s < 8; ++s) {
        const float2 e = block_entry(a, img, x, 4 * g + s / 2);
        v[s] = (s & 1) ? -e.y : e.x;
        v[8 + s] = (s & 1) ? e.x : e.y;
    }
    char* dst = (char*)a.out + off;
    if (a.ct == CT_F32) {
        float4* d = (float4*)dst + lane * 4;
#pragma unroll
        for (int i = 0; i < 4; ++i) d[i] = make_float4(v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]);
    } else {
        uint32_t w[8];
#pragma unroll
        for (int i = 0; i < 8; ++i)
            w[i] = a.ct == CT_BF16 ? pack2<CT_BF16>(v[2 * i], v[2 * i + 1]) : pack2<CT_F16>(v[2 * i], v[2 * i + 1]);
        uint4* d = (uint4*)dst + lane * 2;
        d[0] = make_uint4(w[0], w[1], w[2], w[3]);
        d[1] = make_uint4(w[4], w[5], w[6], w[7]);
    }
}

}  // namespace

hipError_t launch_bfly_images(const void* blocks, void* out, int R, int ct, const FusedTableLayout& L,
                              hipStream_t st) {
    BflyImgArgs a{};
    a.blocks = (const float2*)blocks;
    a.out = out;
    a.R = R;
    a.ct = ct;
    a.rb = (R + 15) / 16;
    a.f1 = L.f1; a.i3 = L.i3; a.f2 = L.f2; a.f3 = L.f3; a.i1 = L.i1; a.i2 = L.i2;
    const int nimg = 2 * a.rb * a.rb + 4 * R;
    hipLaunchKernelGGL(bfly_images_kernel, dim3((unsigned)nimg), dim3(64), 0, st, a);
    return hipGetLastError();
}

}  // namespace lcv
