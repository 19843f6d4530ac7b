/*
 * A stand-in for the HIP runtime API, just large enough to build libxfer's
 * host sources with the host compiler under AddressSanitizer and
 * UndefinedBehaviorSanitizer, with no GPU.  Test infrastructure: the real
 * library is always built against ROCm's own headers.
 *
 * Device memory is host memory here: hipMemcpy copies bytes, events are
 * registered heap objects (a destroy of an unknown handle aborts), streams
 * are opaque tokens never dereferenced.  mock_hip.cpp implements it.
 */
#ifndef XFER_MOCK_HIP_RUNTIME_API_H
#define XFER_MOCK_HIP_RUNTIME_API_H

#include <stddef.h>
#include <stdint.h>

typedef enum hipError_t {
  hipSuccess = 0,
  hipErrorInvalidValue = 1,
  hipErrorOutOfMemory = 2,
  hipErrorNoDevice = 100,
} hipError_t;

typedef struct ihipStream_t *hipStream_t;
typedef struct ihipEvent_t *hipEvent_t;
typedef struct hipGraphExec *hipGraphExec_t;
typedef struct ihipGraph *hipGraph_t;
typedef struct hipGraphNode *hipGraphNode_t;

typedef enum hipMemcpyKind {
  hipMemcpyHostToHost = 0,
  hipMemcpyHostToDevice = 1,
  hipMemcpyDeviceToHost = 2,
  hipMemcpyDeviceToDevice = 3,
  hipMemcpyDefault = 4,
} hipMemcpyKind;

#define hipEventDisableTiming 0x2u

#ifdef __cplusplus
struct dim3 {
  uint32_t x, y, z;
  dim3(uint32_t x_ = 1, uint32_t y_ = 1, uint32_t z_ = 1) : x(x_), y(y_), z(z_) {}
};
typedef struct hipKernelNodeParams {
  dim3 blockDim;
  void **extra;
  void *func;
  dim3 gridDim;
  void **kernelParams;
  unsigned int sharedMemBytes;
} hipKernelNodeParams;
extern "C" {
#endif

hipError_t hipMemcpy(void *dst, const void *src, size_t bytes, hipMemcpyKind kind);
hipError_t hipMemcpyAsync(void *dst, const void *src, size_t bytes, hipMemcpyKind kind, hipStream_t stream);
hipError_t hipEventCreateWithFlags(hipEvent_t *event, unsigned flags);
hipError_t hipEventDestroy(hipEvent_t event);
hipError_t hipEventRecord(hipEvent_t event, hipStream_t stream);
hipError_t hipEventSynchronize(hipEvent_t event);
hipError_t hipStreamWaitEvent(hipStream_t stream, hipEvent_t event, unsigned flags);
hipError_t hipGraphLaunch(hipGraphExec_t exec, hipStream_t stream);
hipError_t hipGraphExecDestroy(hipGraphExec_t exec);
hipError_t hipGraphCreate(hipGraph_t *graph, unsigned flags);
hipError_t hipGraphDestroy(hipGraph_t graph);
hipError_t hipGraphAddMemcpyNode1D(hipGraphNode_t *node, hipGraph_t graph, const hipGraphNode_t *deps, size_t n_deps,
                                   void *dst, const void *src, size_t bytes, hipMemcpyKind kind);
hipError_t hipGraphInstantiateWithFlags(hipGraphExec_t *exec, hipGraph_t graph, unsigned long long flags);
#ifdef __cplusplus
hipError_t hipGraphAddKernelNode(hipGraphNode_t *node, hipGraph_t graph, const hipGraphNode_t *deps, size_t n_deps,
                                 const hipKernelNodeParams *params);
#endif
#ifdef __cplusplus
hipError_t hipLaunchKernel(const void *function, dim3 grid, dim3 block, void **args, size_t lds, hipStream_t stream);
#endif

#ifdef __cplusplus
}
#endif

#endif
