// Wait states a VALU read of an MFMA result needs on this GPU.
//
// Each kernel runs one wave: it sets the accumulator registers v0..v15 to
// 1.0 and the operands to ones, issues one MFMA, waits a fixed number of
// wait states (s_nop n waits n + 1), copies the last result register v15,
// waits long enough for any product to finish, and copies v15 again.  A lane
// whose two copies agree read the finished result.  Every register the
// sequence touches is named in the clobber list, and the only memory access
// is one int per lane into the 64-int output buffer.
//
// Output, one JSON line per kernel:
//   {"mfma": ..., "wait_states": n, "fresh_lanes": lanes that read the result}
#include <hip/hip_runtime.h>

#include <stdio.h>

#define ACC_ONES                                                                                         \
  "v_mov_b32 v0, 1.0\n v_mov_b32 v1, 1.0\n v_mov_b32 v2, 1.0\n v_mov_b32 v3, 1.0\n"                      \
  "v_mov_b32 v4, 1.0\n v_mov_b32 v5, 1.0\n v_mov_b32 v6, 1.0\n v_mov_b32 v7, 1.0\n"                      \
  "v_mov_b32 v8, 1.0\n v_mov_b32 v9, 1.0\n v_mov_b32 v10, 1.0\n v_mov_b32 v11, 1.0\n"                    \
  "v_mov_b32 v12, 1.0\n v_mov_b32 v13, 1.0\n v_mov_b32 v14, 1.0\n v_mov_b32 v15, 1.0\n"
// operand registers v16..v31 (fp8 ones 0x38, or bf16 ones 0x3f80), unit scale in v32
#define OPERANDS(W)                                                                                      \
  "v_mov_b32 v16, " W "\n v_mov_b32 v17, " W "\n v_mov_b32 v18, " W "\n v_mov_b32 v19, " W "\n"          \
  "v_mov_b32 v20, " W "\n v_mov_b32 v21, " W "\n v_mov_b32 v22, " W "\n v_mov_b32 v23, " W "\n"          \
  "v_mov_b32 v24, " W "\n v_mov_b32 v25, " W "\n v_mov_b32 v26, " W "\n v_mov_b32 v27, " W "\n"          \
  "v_mov_b32 v28, " W "\n v_mov_b32 v29, " W "\n v_mov_b32 v30, " W "\n v_mov_b32 v31, " W "\n"          \
  "v_mov_b32 v32, 0x7f7f7f7f\n s_nop 15\n s_nop 15\n"
#define MFMA_F8 "v_mfma_scale_f32_32x32x64_f8f6f4 v[0:15], v[16:23], v[24:31], v[0:15], v32, v32\n"
#define MFMA_BF16 "v_mfma_f32_32x32x16_bf16 v[0:15], v[16:19], v[20:23], v[0:15]\n"
#define SETTLE "s_nop 15\n s_nop 15\n s_nop 15\n s_nop 15\n s_nop 15\n s_nop 15\n s_nop 15\n s_nop 15\n"
#define CLOBBERS                                                                                         \
  "v0", "v1", "v2", "v3", "v4", "v5", "v6", "v7", "v8", "v9", "v10", "v11", "v12", "v13", "v14", "v15", \
      "v16", "v17", "v18", "v19", "v20", "v21", "v22", "v23", "v24", "v25", "v26", "v27", "v28", "v29",   \
      "v30", "v31", "v32"

#define PROBE(NAME, SETUP, MFMA, WAIT)                                                                   \
  __global__ void NAME(int* out) {                                                                       \
    float early, late;                                                                                   \
    asm volatile(ACC_ONES SETUP MFMA WAIT "v_mov_b32 %0, v15\n" SETTLE "v_mov_b32 %1, v15\n"             \
                 : "=v"(early), "=v"(late)                                                               \
                 :                                                                                       \
                 : CLOBBERS);                                                                            \
    out[threadIdx.x] = early == late;                                                                    \
  }

PROBE(f8_19, OPERANDS("0x38383838"), MFMA_F8, "s_nop 15\n s_nop 2\n")
PROBE(f8_20, OPERANDS("0x38383838"), MFMA_F8, "s_nop 15\n s_nop 3\n")
PROBE(f8_24, OPERANDS("0x38383838"), MFMA_F8, "s_nop 15\n s_nop 7\n")
PROBE(bf16_11, OPERANDS("0x3f803f80"), MFMA_BF16, "s_nop 10\n")
PROBE(bf16_12, OPERANDS("0x3f803f80"), MFMA_BF16, "s_nop 11\n")
PROBE(bf16_16, OPERANDS("0x3f803f80"), MFMA_BF16, "s_nop 15\n")

static int run(void (*k)(int*), const char* mfma, int waits, int* dev) {
  int host[64];
  hipLaunchKernelGGL(k, dim3(1), dim3(64), 0, 0, dev);
  if (hipMemcpy(host, dev, sizeof host, hipMemcpyDeviceToHost) != hipSuccess) return 1;
  int fresh = 0;
  for (int i = 0; i < 64; ++i) fresh += host[i];
  printf("{\"mfma\": \"%s\", \"wait_states\": %d, \"fresh_lanes\": %d}\n", mfma, waits, fresh);
  return 0;
}

int main() {
  int* dev = nullptr;
  if (hipMalloc(&dev, 64 * sizeof(int)) != hipSuccess) return 1;
  const char* f8 = "v_mfma_scale_f32_32x32x64_f8f6f4";
  const char* bf = "v_mfma_f32_32x32x16_bf16";
  int err = run(f8_19, f8, 19, dev) | run(f8_20, f8, 20, dev) | run(f8_24, f8, 24, dev) |
            run(bf16_11, bf, 11, dev) | run(bf16_12, bf, 12, dev) | run(bf16_16, bf, 16, dev);
  return err || hipFree(dev) != hipSuccess;
}
