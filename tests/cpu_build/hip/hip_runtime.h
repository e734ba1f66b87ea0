// Host emulation of the HIP runtime header (see simt.h).
#pragma once
#include "../simt.h"
