/* Host-only stand-in (see hip_runtime_api.h): no device code is built with it. */
#ifndef XFER_MOCK_HIP_RUNTIME_H
#define XFER_MOCK_HIP_RUNTIME_H
#include "hip_runtime_api.h"
#define __host__
#define __device__
#endif
