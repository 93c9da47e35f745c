// Issue-rate probes behind the attention kernel's ceilings on gfx950:
//   mfma   v_mfma_f32_32x32x16_bf16 throughput with every SIMD busy
//   exp    v_exp_f32 throughput (the softmax's transcendental)
//   cvt    v_cvt_pk_bf16_f32 throughput (P rounded to bf16 pairs)
//   mixed  one MFMA wave and one exp wave per SIMD side by side
//   inwave every wave issues both: 4 MFMAs and 16 exps per iteration, the
//          exps independent of the MFMAs, in the compiler's order or pinned
//          to MFMA, 4 exps, MFMA, 4 exps, ...
// and the shader clock while the MFMA probe runs (shader-clock counter
// against the 100 MHz real-time counter).  Prints one JSON object per probe.
//
//     magi_rates [--iters N]
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>
#include <cstring>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

#define CHECK(x)                                                                       \
  do {                                                                                 \
    hipError_t e_ = (x);                                                               \
    if (e_ != hipSuccess) {                                                            \
      std::fprintf(stderr, "%s failed: %s\n", #x, hipGetErrorString(e_));              \
      std::exit(1);                                                                    \
    }                                                                                  \
  } while (0)

// Four independent accumulator chains per wave keep the MFMA pipe full.
// clk[0..1] = shader clock at start/end, clk[2..3] = real time (100 MHz),
// taken by lane 0 of the first wave of block 0.
__global__ __launch_bounds__(256) void mfma_probe(int iters, float* sink, long long* clk) {
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(0.001f * (lane + i));
    b[i] = (__bf16)(0.002f * (lane - i));
  }
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  const bool timer = blockIdx.x == 0 && threadIdx.x == 0;
  long long t0 = 0, r0 = 0;
  if (timer) {
    t0 = __builtin_amdgcn_s_memtime();
    r0 = __builtin_amdgcn_s_memrealtime();
  }
  for (int it = 0; it < iters; ++it) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
  }
  if (timer) {
    clk[0] = t0;
    clk[1] = __builtin_amdgcn_s_memtime();
    clk[2] = r0;
    clk[3] = __builtin_amdgcn_s_memrealtime();
  }
  float s = 0.f;
  for (int i = 0; i < 16; ++i) s += c0[i] + c1[i] + c2[i] + c3[i];
  sink[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// Eight independent chains x <- 2^-x per lane (one v_exp_f32 with a negated
// source each; the values stay in [0.5, 1]).
__global__ __launch_bounds__(256) void exp_probe(int iters, float* sink) {
  float x[8];
  for (int i = 0; i < 8; ++i) x[i] = 0.001f * (threadIdx.x + i);
  for (int it = 0; it < iters; ++it)
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = __builtin_amdgcn_exp2f(-x[i]);
  float s = 0.f;
  for (int i = 0; i < 8; ++i) s += x[i];
  sink[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// Eight independent fp32 pair -> packed bf16 conversions per lane; each
// result feeds the next one's input so nothing is hoisted out of the loop.
__global__ __launch_bounds__(256) void cvt_probe(int iters, float* sink) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  float x[8];
  for (int i = 0; i < 8; ++i) x[i] = 1.0f + 0.001f * (threadIdx.x + i);
  for (int it = 0; it < iters; ++it)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const bf16x2 p = __builtin_convertvector((f32x2){x[i], x[(i + 1) & 7]}, bf16x2);
      x[i] = __builtin_bit_cast(float, p);
    }
  float s = 0.f;
  for (int i = 0; i < 8; ++i) s += x[i];
  sink[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// Half the waves run the MFMA loop, half the exp loop, the role alternating
// with the wave index and the block index so that every SIMD (wave w of a
// block goes to SIMD w mod 4) holds both kinds: whether the two pipes
// overlap across waves of one SIMD.
__global__ __launch_bounds__(256) void mixed_probe(int iters, float* sink) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  float s = 0.f;
  if (((wave + blockIdx.x) & 1) == 0) {
    bf16x8 a, b;
    for (int i = 0; i < 8; ++i) {
      a[i] = (__bf16)(0.001f * (lane + i));
      b[i] = (__bf16)(0.002f * (lane - i));
    }
    f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
    for (int it = 0; it < iters; ++it) {
      c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
      c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
      c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
      c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
    }
    for (int i = 0; i < 16; ++i) s += c0[i] + c1[i] + c2[i] + c3[i];
  } else {
    float x[8];
    for (int i = 0; i < 8; ++i) x[i] = 0.001f * (threadIdx.x + i);
    // 16 exp per 4 MFMAs: the softmax's exp count per 32x32 score block
    for (int it = 0; it < 2 * iters; ++it)
#pragma unroll
      for (int i = 0; i < 8; ++i) x[i] = __builtin_amdgcn_exp2f(-x[i]);
    for (int i = 0; i < 8; ++i) s += x[i];
  }
  sink[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// Every wave: 4 MFMAs (independent chains) and 16 exps (8 chains, two
// steps each) per iteration, the exps reading none of the MFMA results.
// PIN fixes the issue order to one MFMA then 4 exps, four times.
template <bool PIN>
__global__ __launch_bounds__(256) void inwave_probe(int iters, float* sink) {
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(0.001f * (lane + i));
    b[i] = (__bf16)(0.002f * (lane - i));
  }
  f32x16 c[4] = {{}, {}, {}, {}};
  float x[8];
  for (int i = 0; i < 8; ++i) x[i] = 0.001f * (threadIdx.x + i);
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      c[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c[j], 0, 0, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i) x[(4 * j + i) & 7] = __builtin_amdgcn_exp2f(-x[(4 * j + i) & 7]);
      if constexpr (PIN) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
        __builtin_amdgcn_sched_group_barrier(0x400, 4, 0);  // then four transcendentals
      }
    }
  }
  float s = 0.f;
  for (int i = 0; i < 16; ++i) s += c[0][i] + c[1][i] + c[2][i] + c[3][i];
  for (int i = 0; i < 8; ++i) s += x[i];
  sink[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

template <typename F>
float time_ms(F launch, int reps) {
  hipEvent_t a, b;
  CHECK(hipEventCreate(&a));
  CHECK(hipEventCreate(&b));
  launch();  // warm-up
  CHECK(hipEventRecord(a, nullptr));
  for (int r = 0; r < reps; ++r) launch();
  CHECK(hipEventRecord(b, nullptr));
  CHECK(hipEventSynchronize(b));
  float ms = 0.f;
  CHECK(hipEventElapsedTime(&ms, a, b));
  CHECK(hipEventDestroy(a));
  CHECK(hipEventDestroy(b));
  return ms / reps;
}

}  // namespace

int main(int argc, char** argv) {
  int iters = 20000;
  for (int i = 1; i + 1 < argc; ++i)
    if (std::strcmp(argv[i], "--iters") == 0) iters = std::atoi(argv[i + 1]);
  hipDeviceProp_t prop;
  CHECK(hipGetDeviceProperties(&prop, 0));
  const int cus = prop.multiProcessorCount;
  // 4 waves per block; 4 blocks per CU = 4 waves per SIMD
  const int blocks = cus * 4;
  float* sink = nullptr;
  long long* clk = nullptr;
  CHECK(hipMalloc(&sink, sizeof(float) * blocks * 256));
  CHECK(hipMalloc(&clk, sizeof(long long) * 4));
  const int reps = 5;

  const float t_mfma = time_ms([&] { hipLaunchKernelGGL(mfma_probe, dim3(blocks), dim3(256), 0, 0, iters, sink, clk); },
                               reps);
  long long c[4];
  CHECK(hipMemcpy(c, clk, sizeof c, hipMemcpyDeviceToHost));
  const double mhz = (double)(c[1] - c[0]) / (double)(c[3] - c[2]) * 100.0;
  const double mfma_flops = (double)blocks * 4 /*waves*/ * iters * 4 /*chains*/ * 32.0 * 32.0 * 16.0 * 2.0;
  const double mfma_tf = mfma_flops / (t_mfma * 1e-3) / 1e12;
  std::printf("{\"probe\": \"mfma_f32_32x32x16_bf16\", \"cus\": %d, \"waves_per_simd\": 4, \"ms\": %.4f, "
              "\"tflops\": %.1f, \"shader_clock_mhz\": %.0f, \"flop_per_clk_per_cu\": %.1f}\n",
              cus, t_mfma, mfma_tf, mhz, mfma_flops / (t_mfma * 1e-3) / (mhz * 1e6) / cus);

  const float t_exp =
      time_ms([&] { hipLaunchKernelGGL(exp_probe, dim3(blocks), dim3(256), 0, 0, iters, sink); }, reps);
  const double exps = (double)blocks * 256 * iters * 8;
  std::printf("{\"probe\": \"v_exp_f32\", \"ms\": %.4f, \"per_s\": %.4e, \"per_clk_per_cu_at_probe_clock\": %.2f}\n",
              t_exp, exps / (t_exp * 1e-3), exps / (t_exp * 1e-3) / (mhz * 1e6) / cus);

  const float t_cvt =
      time_ms([&] { hipLaunchKernelGGL(cvt_probe, dim3(blocks), dim3(256), 0, 0, iters, sink); }, reps);
  const double cvts = (double)blocks * 256 * iters * 8;
  std::printf("{\"probe\": \"v_cvt_pk_bf16_f32\", \"ms\": %.4f, \"per_s\": %.4e, "
              "\"per_clk_per_cu_at_probe_clock\": %.2f}\n",
              t_cvt, cvts / (t_cvt * 1e-3), cvts / (t_cvt * 1e-3) / (mhz * 1e6) / cus);

  // mixed: half the waves of each SIMD on each pipe, each doing the work
  // one pipe alone would do in t_mfma / 2 and t_exp (same iteration count)
  const float t_mix =
      time_ms([&] { hipLaunchKernelGGL(mixed_probe, dim3(blocks), dim3(256), 0, 0, iters, sink); }, reps);
  std::printf("{\"probe\": \"mixed_mfma_exp\", \"ms\": %.4f, \"mfma_alone_half_waves_ms\": %.4f, "
              "\"exp_alone_equiv_ms\": %.4f}\n",
              t_mix, t_mfma / 2, t_exp);
  // in-wave: each wave does the MFMA probe's 4 MFMAs and twice the exp
  // probe's 8 exps per iteration
  const float t_in0 =
      time_ms([&] { hipLaunchKernelGGL(inwave_probe<false>, dim3(blocks), dim3(256), 0, 0, iters, sink); }, reps);
  const float t_in1 =
      time_ms([&] { hipLaunchKernelGGL(inwave_probe<true>, dim3(blocks), dim3(256), 0, 0, iters, sink); }, reps);
  std::printf("{\"probe\": \"inwave_mfma_exp\", \"ms_compiler_order\": %.4f, \"ms_pinned_order\": %.4f, "
              "\"mfma_alone_ms\": %.4f, \"exp_alone_ms\": %.4f}\n",
              t_in0, t_in1, t_mfma, 2 * t_exp);
  CHECK(hipFree(sink));
  CHECK(hipFree(clk));
  return 0;
}
