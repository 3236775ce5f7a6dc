// Host-side driver of the C ABI for AddressSanitizer / UndefinedBehavior-
// Sanitizer builds (the kernels' host code: argument checks, workspace plans
// and layouts). Every entry point is called over a grid of shapes, valid and
// not, with fake, never-dereferenced device pointers. Shapes that pass the
// checks would launch, so they are called only on a host with no HIP device
// (where the call must then report DSA_ERROR_DEVICE). Exit status 0 when
// every status is one the header allows.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <vector>

#include "../../include/dsa.h"

static int failures = 0;
static void expect(bool ok, const char* what, int line) {
  if (!ok) {
    std::fprintf(stderr, "unexpected status: %s (line %d)\n", what, line);
    ++failures;
  }
}
#define EXPECT(c) expect((c), #c, __LINE__)

static bool known(dsa_status_t s) { return s >= DSA_SUCCESS && s <= DSA_ERROR_SCRATCH_LIMIT; }

int main() {
  int ndev = 0;
  if (hipGetDeviceCount(&ndev) != hipSuccess) ndev = 0;
  (void)hipGetLastError();
  void* P = reinterpret_cast<void*>(uintptr_t(1) << 20);  // aligned, never dereferenced
  const int Bs[] = {0, 1, 3, 16, 64, 65535, 65536};
  const int Ns[] = {0, 1, 31, 257, 4096, 32768, 262144, 1 << 24};
  const int ks[] = {-1, 0, 1, 64, 1024, 2048, 4096, 4097};
  const int Hs[] = {0, 1, 8, 64, 65};
  const int Ds[] = {64, 128, 512};
  const int Hqs[] = {8, 16, 128, 144};
  for (int B : Bs)
    for (int N : Ns)
      for (int k : ks) {
        (void)dsa_topk_workspace_bytes(B, N, k, DSA_BF16);
        (void)dsa_topk_workspace_bytes(B, N, k, DSA_F32);
        (void)dsa_indexer_topk_chunks(B, N, k);
        for (int H : Hs) {
          const size_t wi = dsa_indexer_topk_workspace_bytes(B, N, H, k, 1);
          if (wi && ndev == 0) {
            const dsa_status_t s = dsa_indexer_topk(P, P, reinterpret_cast<float*>(P), B, N, H, 128,
                                                    k, reinterpret_cast<int32_t*>(P), nullptr, P,
                                                    wi, nullptr);
            EXPECT(s == DSA_ERROR_DEVICE);
          }
          for (int D : Ds)
            for (int Hq : Hqs) {
              dsa_dims_t d{B, N, H, 128, k, 128, Hq, D, 0.05f};
              const size_t ws = dsa_decode_step_workspace_bytes(&d);
              const size_t wa = dsa_sparse_attend_workspace_bytes(&d);
              (void)dsa_decode_step_mt_workspace_bytes(&d, 2);
              (void)dsa_sparse_attend_mt_workspace_bytes(&d, 4);
              const dsa_status_t s = dsa_decode_step(P, P, reinterpret_cast<float*>(P), P, P, P, P,
                                                     nullptr, &d, P, ws ? ws : 256, nullptr);
              EXPECT(known(s));
              if (ws) EXPECT(s == DSA_ERROR_DEVICE || ndev > 0);
              const dsa_status_t s2 = dsa_decode_step_noalloc(P, P, reinterpret_cast<float*>(P), P,
                                                              P, P, P, nullptr, &d, nullptr);
              EXPECT(known(s2));
              if (ws && ws <= DSA_NOALLOC_SCRATCH_BYTES) EXPECT(s2 == DSA_ERROR_DEVICE || ndev > 0);
              if (ws > DSA_NOALLOC_SCRATCH_BYTES) EXPECT(s2 == DSA_ERROR_SCRATCH_LIMIT);
              const dsa_status_t s3 = dsa_sparse_attend(P, P, reinterpret_cast<int32_t*>(P), P, P,
                                                        &d, P, wa ? wa : 256, nullptr);
              EXPECT(known(s3));
              if (ndev > 0) continue;  // everything below would launch
              EXPECT(dsa_decode_step_ragged(P, P, reinterpret_cast<float*>(P), P, P, P,
                                            reinterpret_cast<int32_t*>(P), P, nullptr, &d, P,
                                            ws ? ws : 256, nullptr) == s);
            }
        }
      }
  // Errors with null pointers and zero sizes, whatever the device.
  EXPECT(dsa_indexer_score(nullptr, P, reinterpret_cast<float*>(P), reinterpret_cast<float*>(P), 1,
                           1, 1, 128, nullptr) == DSA_ERROR_INVALID_VALUE);
  EXPECT(dsa_topk(P, DSA_F32, 1, 10, 11, reinterpret_cast<int32_t*>(P), nullptr, 0, P, 1 << 20,
                  nullptr) == DSA_ERROR_INVALID_VALUE);
  EXPECT(dsa_compress(P, reinterpret_cast<float*>(P), P, 1, 1, 100, nullptr) ==
         DSA_ERROR_NOT_SUPPORTED);
  EXPECT(dsa_indexer_qproj(P, P, P, 1, 100, 1, 128, nullptr) == DSA_ERROR_NOT_SUPPORTED);
  // 0..7 all lie in the enum's range (7 is no status: the unknown-code name).
  for (int s = 0; s < 8; ++s) EXPECT(dsa_status_string(static_cast<dsa_status_t>(s)) != nullptr);
  std::printf("abi driver: %d unexpected statuses, %d devices\n", failures, ndev);
  return failures ? 1 : 0;
}
