// Host-side launchers of the gfx950 MoE layer kernels (internal to the library).
#pragma once

#include "common.h"

namespace moe {

// Decode path, B = 1..8.  route_only: only the router + selection kernel.
hipError_t launch_decode(int B, int fmt, bool route_only, const uint16_t* x, const uint16_t* rw,
                         const ExpertsDev& routed, const ExpertsDev& shared, uint16_t* out,
                         int32_t* ids, float* w, uint8_t* ws, hipStream_t st);

// The same path as three launches (route, gate/up, down).
hipError_t launch_decode_split(int B, int fmt, const uint16_t* x, const uint16_t* rw,
                               const ExpertsDev& routed, const ExpertsDev& shared, uint16_t* out,
                               int32_t* ids, float* w, uint8_t* ws, hipStream_t st);

// Fused single-launch decode path, B = 1..8 (needs 256 co-resident workgroups).
// With both events given, the launch records the kernel's own start and end
// on them (hipExtLaunchKernel).
bool fused_supported();
hipError_t launch_decode_fused(int B, int fmt, const uint16_t* x, const uint16_t* rw,
                               const ExpertsDev& routed, const ExpertsDev& shared, uint16_t* out,
                               int32_t* ids, float* w, uint8_t* ws, hipStream_t st,
                               hipEvent_t ev_start = nullptr, hipEvent_t ev_stop = nullptr,
                               const FuseDev& fuse = FuseDev{});

// The same single-launch layer with two shared experts (NVFP4, Flint's shape
// otherwise; no fused neighbours).
bool fused_ns2_supported();
hipError_t launch_decode_fused_ns2(int B, const uint16_t* x, const uint16_t* rw,
                                   const ExpertsDev& routed, const ExpertsDev& shared,
                                   uint16_t* out, int32_t* ids, float* w, uint8_t* ws,
                                   hipStream_t st, hipEvent_t ev_start = nullptr,
                                   hipEvent_t ev_stop = nullptr);

// The same single-launch layer in W4A4 (NVFP4 weights, NVFP4 activations
// with the Four Over Six block scale), Flint's shape, batch 1 to 8.
bool fused_a4_supported(int B);
hipError_t launch_a4_convert_check(unsigned long long* counts, hipStream_t st);
hipError_t launch_decode_fused_a4(int B, const uint16_t* x, const uint16_t* rw,
                                  const ExpertsDev& routed, const ExpertsDev& shared, uint16_t* out,
                                  int32_t* ids, float* w, uint8_t* ws, hipStream_t st,
                                  hipEvent_t ev_start = nullptr, hipEvent_t ev_stop = nullptr);

// A stack of L layers (same x) in one launch of the fused kernel's body.
hipError_t launch_decode_stack(int B, int fmt, const uint16_t* x, const LayerDev* layers, int L,
                               uint16_t* out, int32_t* ids, uint8_t* ws, hipStream_t st);

// A chained residual stack in one launch: x_{l+1} = x_l + layer_l(norm_l(x_l)),
// out[l] = x_{l+1}; norm_w bf16 [L][H] (nullptr: no norm).
hipError_t launch_decode_chain(int B, int fmt, const uint16_t* x, const LayerDev* layers, int L,
                               const uint16_t* norm_w, float eps, uint16_t* out, int32_t* ids,
                               uint8_t* ws, hipStream_t st);

// Copy the workspace's wait-status word to *status (device) and clear it.
hipError_t launch_ws_status(uint8_t* ws, int32_t* status, hipStream_t st);

// Dense NVFP4 GEMV, B = 1..8, K % 32 == 0, K <= 8192, B * K <= 32768.
constexpr int kGemvMaxK = 8192;
constexpr int kGemvMaxBK = 32768;                  // x staged in LDS: B * K * 2 bytes <= 64 KiB
hipError_t launch_nvfp4_gemv(int B, int K, int N, const uint16_t* x, const uint8_t* codes,
                             const uint8_t* scales, const float* glob, uint16_t* y,
                             hipStream_t st);

// Parity probe: one NVFP4 tensor [rows][cols] decoded to fp32.
hipError_t launch_dequant(const uint8_t* codes, const uint8_t* scales, const float* glob, int rows,
                          int cols, float* out, hipStream_t st);

// Prefill path, T >= 1 tokens.
hipError_t launch_prefill(int T, int fmt, const uint16_t* x, const uint16_t* rw,
                          const ExpertsDev& routed, const ExpertsDev& shared, uint16_t* out,
                          int32_t* ids, float* w, uint8_t* ws, hipStream_t st,
                          const FuseDev& fuse = FuseDev{});

// General-shape decode path, B = 1..8 (any served shape and format,
// including MXFP8): four launches.  The route-only entry runs its first two.
size_t gen_ws_bytes(const GenShape& S);
hipError_t launch_route_general(int B, const GenShape& S, const uint16_t* x, const uint16_t* rw,
                                int32_t* ids, float* w, uint8_t* ws, hipStream_t st, int a4 = 0);
hipError_t launch_decode_general(int B, int fmt, const GenShape& S, const uint16_t* x,
                                 const uint16_t* rw, const ExpertsDev& routed,
                                 const ExpertsDev& shared, uint16_t* out, int32_t* ids, float* w,
                                 uint8_t* ws, hipStream_t st);

// Workspace bytes of the prefill path for T tokens (0 = not served).
size_t prefill_ws_bytes(int T);

}  // namespace moe
