// Host emulation of the HIP runtime API header (see simt.h).
#pragma once
#include "../simt.h"
